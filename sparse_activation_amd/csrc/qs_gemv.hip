// Gather-GEMV kernels of the sparse-activation linear (gfx950).
//
// y[r, o] = sum over selected j of xs[r, j] * W^T[j, o]
//
// Q-Sparse news article (zxwl-tech.com), section "Sparsification with the
// Top-K function": X (.) M replaces X in Y = X . W^T, so only the rows of
// W^T whose input feature survives the top-K contribute; Q-Sparse aibase
// report: memory traffic is the inference bottleneck.  These kernels read
// exactly those rows: for a batch, the union over its tokens, each row once.
//
// Work decomposition (grid = column tiles x K-splits x token tiles):
//   * a workgroup owns a range of `cand` candidate input rows of one split;
//     it loads the sparsified activations xs of its token tile for that
//     range, and one wavefront ballot per 64 candidates compacts the rows
//     that some token selects into an LDS list (ascending);
//   * each half-wavefront streams one selected W^T row segment per step
//     with 16-byte loads (512 contiguous bytes per row per instruction),
//     four rows in flight per lane, and accumulates into fp32 registers;
//   * the eight row slots of the workgroup are summed in LDS in a fixed
//     order, the split's partial tile goes to the workspace, and the last
//     workgroup of each column tile (device-scope counter) sums the splits
//     in split order, applies the epilogue and stores y.  No floating-point
//     atomics: the result is bitwise reproducible.
//
// The ternary x int8 variant does the same with 2-bit packed weights and
// exact int32 accumulation.
#include "qs_internal.h"

namespace qs {
namespace {

constexpr int kNT = 256;     // threads per workgroup
constexpr int kLPR = 32;     // lanes per weight-row segment
constexpr int kRPI = 64 / kLPR;
constexpr int kNSlot = 4 * kRPI;
constexpr int kUnroll = 4;
constexpr int kTargetWG = 1024;

__device__ __forceinline__ uint32_t popc_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

template <int WBF16>
__device__ __forceinline__ void unpack(const uint4& v, float* w) {
    if constexpr (WBF16) {
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[2 * i] = __uint_as_float(u[i] << 16);
            w[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
        }
    } else {
        w[0] = __uint_as_float(v.x);
        w[1] = __uint_as_float(v.y);
        w[2] = __uint_as_float(v.z);
        w[3] = __uint_as_float(v.w);
    }
}

__device__ __forceinline__ void store_final(const GemvArgs& a, int64_t i, float s) {
    if (a.epilogue == EPI_RELU2) {
        reinterpret_cast<float*>(a.y)[i] = s > 0.0f ? __fmul_rn(s, s) : 0.0f;
    } else if (a.y_bf16) {
        reinterpret_cast<uint16_t*>(a.y)[i] = f32_to_bf16_rne(s);
    } else {
        reinterpret_cast<float*>(a.y)[i] = s;
    }
}

template <int WBF16, int BT>
__global__ __launch_bounds__(kNT) void gather_gemv_kernel(GemvArgs a, int cand, int nsplit) {
    constexpr int EPT = WBF16 ? 8 : 4;
    constexpr int CT = kLPR * EPT;
    constexpr int TG = BT < 2 ? BT : 2;
    extern __shared__ float smem[];
    float* s_coef = smem;                                  // [cand][BT]
    int* s_act = reinterpret_cast<int*>(smem + (size_t)cand * BT);   // [cand]
    __shared__ int s_wcnt[4];
    __shared__ int s_last;

    const int tile = blockIdx.x, split = blockIdx.y, tt = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t rows = a.rows, d_in = a.d_in, n_out = a.n_out;
    const int64_t j0 = (int64_t)split * cand;
    const int64_t j1 = min(d_in, j0 + (int64_t)cand);
    const int64_t tok0 = (int64_t)tt * BT;

    // Phase A: selected candidate rows (union over the token tile), ascending.
    int nact = 0;
    for (int64_t c0 = j0; c0 < j1; c0 += kNT) {
        const int64_t j = c0 + tid;
        float c[BT];
        bool any = false;
#pragma unroll
        for (int t = 0; t < BT; ++t) {
            float v = 0.0f;
            if (j < j1 && tok0 + t < rows) v = a.xs[(tok0 + t) * d_in + j];
            c[t] = v;
            any = any || (v != 0.0f);
        }
        const uint64_t b = __ballot(any);
        if (lane == 0) s_wcnt[wave] = (int)__popcll(b);
        __syncthreads();
        int before = nact, total = nact;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if (w < wave) before += s_wcnt[w];
            total += s_wcnt[w];
        }
        if (any) {
            const int pos = before + (int)popc_below(b);
            s_act[pos] = (int)j;
#pragma unroll
            for (int t = 0; t < BT; ++t) s_coef[pos * BT + t] = c[t];
        }
        nact = total;
        __syncthreads();
    }

    // Phase B: stream the selected W^T row segments.
    const int slot = wave * kRPI + lane / kLPR;
    const int64_t col = (int64_t)tile * CT + (lane % kLPR) * EPT;
    const bool colok = col < n_out;
    const int64_t esize = WBF16 ? 2 : 4;
    const char* wcol = reinterpret_cast<const char*>(a.w) + col * esize;
    const int64_t rowbytes = n_out * esize;

    float acc[BT][EPT];
#pragma unroll
    for (int t = 0; t < BT; ++t)
#pragma unroll
        for (int e = 0; e < EPT; ++e) acc[t][e] = 0.0f;

    for (int a0 = slot; a0 < nact; a0 += kNSlot * kUnroll) {
        uint4 wv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int ai = a0 + u * kNSlot;
            if (ai < nact && colok)
                wv[u] = *reinterpret_cast<const uint4*>(wcol + (int64_t)s_act[ai] * rowbytes);
            else
                wv[u] = make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int ai = a0 + u * kNSlot;
            if (ai < nact) {
                float w[EPT];
                unpack<WBF16>(wv[u], w);
#pragma unroll
                for (int t = 0; t < BT; ++t) {
                    const float c = s_coef[ai * BT + t];
#pragma unroll
                    for (int e = 0; e < EPT; ++e) acc[t][e] = fmaf(c, w[e], acc[t][e]);
                }
            }
        }
    }
    __syncthreads();   // s_coef / s_act are dead from here: reuse as the reduction buffer

    // Phase C: sum the row slots in slot order, token group by token group.
    float* s_red = smem;   // [kNSlot][TG][CT]
    const int cl = (lane % kLPR) * EPT;
#pragma unroll
    for (int t0 = 0; t0 < BT; t0 += TG) {
#pragma unroll
        for (int g = 0; g < TG; ++g)
#pragma unroll
            for (int e = 0; e < EPT; ++e) s_red[(slot * TG + g) * CT + cl + e] = acc[t0 + g][e];
        __syncthreads();
        for (int o = tid; o < TG * CT; o += kNT) {
            float s = 0.0f;
#pragma unroll
            for (int sl = 0; sl < kNSlot; ++sl) s += s_red[sl * TG * CT + o];
            const int64_t row = tok0 + t0 + o / CT;
            const int64_t cg = (int64_t)tile * CT + (o % CT);
            if (row < rows && cg < n_out) {
                if (nsplit == 1) store_final(a, row * n_out + cg, s);
                else a.partial[((int64_t)split * rows + row) * n_out + cg] = s;
            }
        }
        __syncthreads();
    }

    // Phase D: the last split of this tile sums the partials in split order.
    if (nsplit > 1) {
        __threadfence();
        __syncthreads();
        const int ci = tt * gridDim.x + tile;
        if (tid == 0) s_last = (atomicAdd(&a.counters[ci], 1) == nsplit - 1);
        __syncthreads();
        if (s_last) {
            __threadfence();
            for (int o = tid; o < BT * CT; o += kNT) {
                const int64_t row = tok0 + o / CT;
                const int64_t cg = (int64_t)tile * CT + (o % CT);
                if (row < rows && cg < n_out) {
                    float s = 0.0f;
                    for (int sp = 0; sp < nsplit; ++sp)
                        s += a.partial[((int64_t)sp * rows + row) * n_out + cg];
                    store_final(a, row * n_out + cg, s);
                }
            }
            if (tid == 0) a.counters[ci] = 0;
        }
    }
}

int pow2_tile(int64_t rows, int cap) {
    int bt = 1;
    while (bt < rows && bt < cap) bt *= 2;
    return bt;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- ternary x int8

constexpr int kI8EPT = 32;                 // columns per lane (8 bytes of packed weights)
constexpr int kI8CT = kLPR * kI8EPT;       // 1024 columns per tile
constexpr int kI8TargetWG = 512;

template <int BT>
__global__ __launch_bounds__(kNT) void i8t_gemv_kernel(I8tArgs a, int cand, int nsplit) {
    extern __shared__ int ismem[];
    int* s_coef = ismem;                        // [cand][BT]
    int* s_act = ismem + (size_t)cand * BT;     // [cand]
    __shared__ int s_wcnt[4];
    __shared__ int s_last;

    const int tile = blockIdx.x, split = blockIdx.y, tt = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t rows = a.rows, d_in = a.d_in, n_out = a.n_out;
    const int64_t j0 = (int64_t)split * cand;
    const int64_t j1 = min(d_in, j0 + (int64_t)cand);
    const int64_t tok0 = (int64_t)tt * BT;

    int nact = 0;
    for (int64_t c0 = j0; c0 < j1; c0 += kNT) {
        const int64_t j = c0 + tid;
        int c[BT];
        bool any = false;
#pragma unroll
        for (int t = 0; t < BT; ++t) {
            int v = 0;
            if (j < j1 && tok0 + t < rows) v = a.qs[(tok0 + t) * d_in + j];
            c[t] = v;
            any = any || (v != 0);
        }
        const uint64_t b = __ballot(any);
        if (lane == 0) s_wcnt[wave] = (int)__popcll(b);
        __syncthreads();
        int before = nact, total = nact;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if (w < wave) before += s_wcnt[w];
            total += s_wcnt[w];
        }
        if (any) {
            const int pos = before + (int)popc_below(b);
            s_act[pos] = (int)j;
#pragma unroll
            for (int t = 0; t < BT; ++t) s_coef[pos * BT + t] = c[t];
        }
        nact = total;
        __syncthreads();
    }

    const int slot = wave * kRPI + lane / kLPR;
    const int64_t col = (int64_t)tile * kI8CT + (lane % kLPR) * kI8EPT;
    const bool colok = col < n_out;
    const bool col2ok = col + 16 < n_out;     // n_out % 16 == 0: second word present
    const int64_t rowbytes = n_out / 4;
    const uint8_t* wcol = a.wt + col / 4;

    int acc[BT][kI8EPT];
#pragma unroll
    for (int t = 0; t < BT; ++t)
#pragma unroll
        for (int e = 0; e < kI8EPT; ++e) acc[t][e] = 0;

    for (int a0 = slot; a0 < nact; a0 += kNSlot * kUnroll) {
        uint2 wv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int ai = a0 + u * kNSlot;
            // Two 4-byte loads: rows are only 4-byte aligned when n_out % 32 != 0.
            wv[u] = make_uint2(0u, 0u);
            if (ai < nact && colok) {
                const uint32_t* p =
                    reinterpret_cast<const uint32_t*>(wcol + (int64_t)s_act[ai] * rowbytes);
                wv[u].x = p[0];
                if (col2ok) wv[u].y = p[1];
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int ai = a0 + u * kNSlot;
            if (ai < nact) {
                int c[BT];
#pragma unroll
                for (int t = 0; t < BT; ++t) c[t] = s_coef[ai * BT + t];
#pragma unroll
                for (int e = 0; e < kI8EPT; ++e) {
                    const uint32_t word = e < 16 ? wv[u].x : wv[u].y;
                    // 2-bit two's complement field: 00 -> 0, 01 -> +1, 11 -> -1
                    const int tv = __builtin_amdgcn_sbfe((int)word, (2 * e) & 31, 2);
#pragma unroll
                    for (int t = 0; t < BT; ++t) acc[t][e] += c[t] * tv;
                }
            }
        }
    }
    __syncthreads();

    // Integer partial sums are exact, so only the epilogue needs an order.
    int* s_red = ismem;   // [kNSlot][CT] per token
    const int cl = (lane % kLPR) * kI8EPT;
#pragma unroll
    for (int t = 0; t < BT; ++t) {
#pragma unroll
        for (int e = 0; e < kI8EPT; ++e) s_red[slot * kI8CT + cl + e] = acc[t][e];
        __syncthreads();
        for (int o = tid; o < kI8CT; o += kNT) {
            int s = 0;
#pragma unroll
            for (int sl = 0; sl < kNSlot; ++sl) s += s_red[sl * kI8CT + o];
            const int64_t row = tok0 + t;
            const int64_t cg = (int64_t)tile * kI8CT + o;
            if (row < rows && cg < n_out) {
                if (nsplit == 1) {
                    if (a.acc) a.acc[row * n_out + cg] = s;
                    if (a.y) a.y[row * n_out + cg] =
                        __fmul_rn((float)s, __fdiv_rn(a.alpha, a.xscale[row]));
                } else {
                    a.partial[((int64_t)split * rows + row) * n_out + cg] = s;
                }
            }
        }
        __syncthreads();
    }

    if (nsplit > 1) {
        __threadfence();
        __syncthreads();
        const int ci = tt * gridDim.x + tile;
        if (tid == 0) s_last = (atomicAdd(&a.counters[ci], 1) == nsplit - 1);
        __syncthreads();
        if (s_last) {
            __threadfence();
            for (int o = tid; o < BT * kI8CT; o += kNT) {
                const int64_t row = tok0 + o / kI8CT;
                const int64_t cg = (int64_t)tile * kI8CT + (o % kI8CT);
                if (row < rows && cg < n_out) {
                    int s = 0;
                    for (int sp = 0; sp < nsplit; ++sp)
                        s += a.partial[((int64_t)sp * rows + row) * n_out + cg];
                    if (a.acc) a.acc[row * n_out + cg] = s;
                    if (a.y) a.y[row * n_out + cg] =
                        __fmul_rn((float)s, __fdiv_rn(a.alpha, a.xscale[row]));
                }
            }
            if (tid == 0) a.counters[ci] = 0;
        }
    }
}

}  // namespace

GemvPlan plan_gemv(int64_t rows, int64_t d_in, int64_t n_out, int w_is_bf16) {
    GemvPlan p{};
    p.lpr = kLPR;
    p.ept = w_is_bf16 ? 8 : 4;
    p.ct = p.lpr * p.ept;
    p.n_tiles = (int)ceil_div(n_out, p.ct);
    p.bt = pow2_tile(rows, 16);
    p.n_tok_tiles = (int)ceil_div(rows, p.bt);
    const int cand_max = 8192 / p.bt < 2048 ? 8192 / p.bt : 2048;   // <= 32 KB of coefficients
    const int64_t base = (int64_t)p.n_tiles * p.n_tok_tiles;
    int64_t ns = ceil_div(kTargetWG, base);
    if (ns < 1) ns = 1;
    int64_t cand = ceil_div(ceil_div(d_in, ns), 64) * 64;
    if (cand > cand_max) cand = cand_max;
    if (cand < 64) cand = 64;
    p.cand = (int)cand;
    p.nsplit = (int)ceil_div(d_in, cand);
    if (p.nsplit < 1) p.nsplit = 1;
    p.partial_floats = p.nsplit > 1 ? (size_t)p.nsplit * rows * n_out : 0;
    p.n_counters = p.n_tiles * p.n_tok_tiles;
    return p;
}

hipError_t launch_gemv(const GemvPlan& p, int w_is_bf16, const GemvArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    const int ept = w_is_bf16 ? 8 : 4;
    const int ct = kLPR * ept;
    const int tg = p.bt < 2 ? p.bt : 2;
    size_t lds_a = (size_t)p.cand * p.bt * 4 + (size_t)p.cand * 4;
    size_t lds_c = (size_t)kNSlot * tg * ct * 4;
    size_t lds = lds_a > lds_c ? lds_a : lds_c;
    dim3 grid(p.n_tiles, p.nsplit, p.n_tok_tiles);
#define QS_GEMV_CASE(WB, BTV)                                                              \
    if (w_is_bf16 == WB && p.bt == BTV) {                                                  \
        gather_gemv_kernel<WB, BTV><<<grid, dim3(kNT), lds, stream>>>(a, p.cand, p.nsplit); \
        return hipGetLastError();                                                          \
    }
    QS_GEMV_CASE(1, 1) QS_GEMV_CASE(1, 2) QS_GEMV_CASE(1, 4) QS_GEMV_CASE(1, 8) QS_GEMV_CASE(1, 16)
    QS_GEMV_CASE(0, 1) QS_GEMV_CASE(0, 2) QS_GEMV_CASE(0, 4) QS_GEMV_CASE(0, 8) QS_GEMV_CASE(0, 16)
#undef QS_GEMV_CASE
    return hipErrorInvalidValue;
}

I8tPlan plan_i8t(int64_t rows, int64_t d_in, int64_t n_out) {
    I8tPlan p{};
    p.ct = kI8CT;
    p.n_tiles = (int)ceil_div(n_out, p.ct);
    p.bt = pow2_tile(rows, 4);
    p.n_tok_tiles = (int)ceil_div(rows, p.bt);
    const int cand_max = 4096 / p.bt;
    const int64_t base = (int64_t)p.n_tiles * p.n_tok_tiles;
    int64_t ns = ceil_div(kI8TargetWG, base);
    if (ns < 1) ns = 1;
    int64_t cand = ceil_div(ceil_div(d_in, ns), 64) * 64;
    if (cand > cand_max) cand = cand_max;
    if (cand < 64) cand = 64;
    p.cand = (int)cand;
    p.nsplit = (int)ceil_div(d_in, cand);
    if (p.nsplit < 1) p.nsplit = 1;
    p.partial_ints = p.nsplit > 1 ? (size_t)p.nsplit * rows * n_out : 0;
    p.n_counters = p.n_tiles * p.n_tok_tiles;
    return p;
}

hipError_t launch_i8t(const I8tPlan& p, const I8tArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    size_t lds_a = (size_t)p.cand * p.bt * 4 + (size_t)p.cand * 4;
    size_t lds_c = (size_t)kNSlot * kI8CT * 4;
    size_t lds = lds_a > lds_c ? lds_a : lds_c;
    dim3 grid(p.n_tiles, p.nsplit, p.n_tok_tiles);
#define QS_I8T_CASE(BTV)                                                                \
    if (p.bt == BTV) {                                                                  \
        i8t_gemv_kernel<BTV><<<grid, dim3(kNT), lds, stream>>>(a, p.cand, p.nsplit);    \
        return hipGetLastError();                                                       \
    }
    QS_I8T_CASE(1) QS_I8T_CASE(2) QS_I8T_CASE(4)
#undef QS_I8T_CASE
    return hipErrorInvalidValue;
}

}  // namespace qs
