// MFMA kernels (gfx950): the dense bf16 GEMM behind the batched (prefill)
// sparse linear, the fused dReLU gate/up projection of the Turbo Sparse FFN,
// and the nonzero compaction of the FFN intermediate.
#include "qs_internal.h"

namespace qs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t popc_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
    return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------
// Dense NT GEMM  C[M, N] = A[M, K] . B[N, K]^T  (bf16 in, fp32 accumulate).
//
// Q-Sparse news article (zxwl-tech.com), section "Sparsification with the
// Top-K function": every projection is Y = X . W^T with X replaced by
// X (.) M.  For a large token batch the union of the per-token selections
// covers every input feature of a tile, so the product is a real dense
// contraction; A is X (.) M, written in bf16 by the selection kernel.
//
// Tile BM x BN x 32 per workgroup, WM x WN wavefronts each owning a 128 x 64
// block of 32x32x16 MFMA tiles.  LDS holds one BK = 32 slice of A and B in
// 16-byte chunks, XOR-swizzled per row pair so the fragment reads
// (32 rows x one chunk) hit distinct banks; the next slice is prefetched into
// registers while the MFMAs run.  Tiles are ordered XCD by XCD (the
// dispatcher places workgroup b on XCD b % 8), each XCD walking a contiguous
// range of tiles that share rows of A and B in its L2.
// ---------------------------------------------------------------------------

constexpr int kBK = 32;

__device__ __forceinline__ int swz(int row, int kc) { return row * 4 + (kc ^ ((row >> 1) & 3)); }

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_nt_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, void* __restrict__ C,
    int M, int N, int K, int c_bf16, int tiles_m, int tiles_n) {
    constexpr int NTH = 64 * WM * WN;
    constexpr int TM = BM / WM / 32;   // MFMA tiles per wave along M
    constexpr int TN = BN / WN / 32;   // along N
    static_assert(TM * 32 * WM == BM && TN * 32 * WN == BN, "tile shape");
    __shared__ u32x4 sA[BM * 4];
    __shared__ u32x4 sB[BN * 4];

    // ---- tile order: contiguous range per XCD, grouped along M inside it.
    const int ntiles = tiles_m * tiles_n;
    int tile = blockIdx.x;
    if (ntiles % 8 == 0) tile = (blockIdx.x % 8) * (ntiles / 8) + blockIdx.x / 8;
    constexpr int GM = 8;
    const int group = tile / (GM * tiles_n);
    const int first_m = group * GM;
    const int gm = min(GM, tiles_m - first_m);
    const int tm = first_m + (tile % (GM * tiles_n)) % gm;
    const int tn = (tile % (GM * tiles_n)) / gm;
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    constexpr int CA = (BM * 4 + NTH - 1) / NTH;   // 16-byte chunks per thread
    constexpr int CB = (BN * 4 + NTH - 1) / NTH;
    u32x4 ra[CA], rb[CB];
    const u32x4 zero = {0u, 0u, 0u, 0u};

    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int c = tid + i * NTH;
            const int row = c >> 2, gk = k0 + (c & 3) * 8;
            const int gr = m0 + row;
            ra[i] = (c < BM * 4 && gr < M && gk < K)
                        ? *reinterpret_cast<const u32x4*>(A + (int64_t)gr * K + gk) : zero;
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int c = tid + i * NTH;
            const int row = c >> 2, gk = k0 + (c & 3) * 8;
            const int gr = n0 + row;
            rb[i] = (c < BN * 4 && gr < N && gk < K)
                        ? *reinterpret_cast<const u32x4*>(B + (int64_t)gr * K + gk) : zero;
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int c = tid + i * NTH;
            if (c < BM * 4) sA[swz(c >> 2, c & 3)] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int c = tid + i * NTH;
            if (c < BN * 4) sB[swz(c >> 2, c & 3)] = rb[i];
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    gload(0);
    lstore();
    __syncthreads();
    const int r32 = lane & 31, kg = lane >> 5;
    for (int k0 = 0; k0 < K; k0 += kBK) {
        const bool more = k0 + kBK < K;
        if (more) gload(k0 + kBK);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int kc = ks * 2 + kg;          // 8-element chunk of this lane's k group
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = as_bf16x8(sA[swz(wm * TM * 32 + i * 32 + r32, kc)]);
#pragma unroll
            for (int j = 0; j < TN; ++j) bfr[j] = as_bf16x8(sB[swz(wn * TN * 32 + j * 32 + r32, kc)]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
        if (more) lstore();
        __syncthreads();
    }

    // ---- epilogue: acc[i][j][v] is C[row, col] with
    //      row = 8 (v / 4) + 4 (lane / 32) + v % 4, col = lane % 32 (within the 32x32 tile)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * TN * 32 + j * 32 + r32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm * TM * 32 + i * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
                if (row < M && col < N) {
                    const int64_t o = (int64_t)row * N + col;
                    if (c_bf16) reinterpret_cast<uint16_t*>(C)[o] = f32_to_bf16_rne(acc[i][j][v]);
                    else reinterpret_cast<float*>(C)[o] = acc[i][j][v];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dReLU gate/up (Turbo Sparse summary, Eq. 2: ReLU after both the gate and the
// up projection, so h = relu(g) * relu(u) is zero wherever g <= 0).
//
// One workgroup owns 16 neurons; its four wavefronts split the model
// dimension (k-steps of 32 dealt round-robin) and each computes a 16 tokens x
// 16 neurons partial product with v_mfma_f32_16x16x32_bf16 (A = tokens, rows
// past the batch are zero and load nothing; B = 16 rows of W).  The partials
// are summed in LDS in wave order, the bias is added, and the up projection
// is then computed only for neurons with g > 0 for some token of the tile:
// lanes of inactive neurons issue no loads, so the rows of W_up of inactive
// neurons are never read.
// ---------------------------------------------------------------------------

constexpr int kDreluUnroll = 8;

// w_tile = the workgroup's first neuron row, n_tile = neurons of the tile that
// exist (both uniform); lanes with load_w == false read zeros.
__device__ __forceinline__ void drelu_partial(const uint16_t* __restrict__ x, int64_t rows,
                                              int64_t tok0, int64_t d,
                                              const uint16_t* __restrict__ w_tile, int64_t n_tile,
                                              bool load_w, int wave, int lane, f32x4& acc) {
    // Buffer views: loads never branch, and rows past the batch, lanes of
    // inactive neurons and k past the row end read zero.
    const int r16 = lane & 15, kg = lane >> 4;
    constexpr uint32_t kOff = 0x40000000u;   // out of range for both views
    const int64_t ntok = min((int64_t)16, rows - tok0);
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x + tok0 * d), (short)0, (int)(ntok * d * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(w_tile), (short)0, (int)(n_tile * d * 2), 0x00020000);
    const uint32_t xrow = (uint32_t)(r16 * d * 2);   // this lane's token row / neuron row
    const int nsteps = (int)((d + 31) / 32);
    for (int s0 = wave; s0 < nsteps; s0 += 4 * kDreluUnroll) {
        u32x4 av[kDreluUnroll], bv[kDreluUnroll];
#pragma unroll
        for (int u = 0; u < kDreluUnroll; ++u) {
            const int s = s0 + 4 * u;
            const int64_t k = (int64_t)s * 32 + kg * 8;
            const bool in = s < nsteps && k < d;
            av[u] = __builtin_amdgcn_raw_buffer_load_b128(xrs, in ? xrow + (uint32_t)(k * 2) : kOff, 0, 0);
            bv[u] = __builtin_amdgcn_raw_buffer_load_b128(
                wrs, in && load_w ? xrow + (uint32_t)(k * 2) : kOff, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kDreluUnroll; ++u)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[u]), as_bf16x8(bv[u]), acc,
                                                          0, 0, 0);
    }
}

__global__ __launch_bounds__(256) void drelu_gate_up_kernel(DreluArgs a) {
    __shared__ f32x4 s_part[4][64];
    __shared__ uint32_t s_act;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, kg = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t rows = a.rows, d = a.d, ffn = a.ffn;
    const int64_t n = n0 + r16;                 // this lane's neuron (B column / D column)
    const bool n_ok = n < ffn;

    if (blockIdx.x == 0 && a.zero_ptr != nullptr)
        for (int i = tid; i < a.n_zero; i += 256) a.zero_ptr[i] = 0;

    for (int64_t tok0 = 0; tok0 < rows; tok0 += 16) {
        // gate partials
        const int64_t n_tile = min((int64_t)16, ffn - n0);
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        drelu_partial(a.x, rows, tok0, d, a.wg + n0 * d, n_tile, n_ok, wave, lane, acc);
        s_part[wave][lane] = acc;
        __syncthreads();
        f32x4 g = s_part[0][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) g += s_part[w][lane];
        const float bg = (a.bg != nullptr && n_ok) ? a.bg[n] : 0.0f;
        bool pos = false;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            g[v] = g[v] + bg;
            const int64_t tok = tok0 + 4 * kg + v;   // D row = token
            pos = pos || (tok < rows && n_ok && g[v] > 0.0f);
        }
        const uint64_t bal = __ballot(pos);
        const uint32_t act = (uint32_t)((bal | (bal >> 16) | (bal >> 32) | (bal >> 48)) & 0xFFFFu);
        __syncthreads();   // s_part reused below

        f32x4 u = {0.0f, 0.0f, 0.0f, 0.0f};
        if (act != 0u) {   // uniform: every wave computes the same ballot
            const bool mine = ((act >> r16) & 1u) != 0u;
            drelu_partial(a.x, rows, tok0, d, a.wu + n0 * d, n_tile, mine, wave, lane, u);
            s_part[wave][lane] = u;
            __syncthreads();
            u = s_part[0][lane];
#pragma unroll
            for (int w = 1; w < 4; ++w) u += s_part[w][lane];
            __syncthreads();
        }
        if (wave == 0 && n_ok) {
            const float bu = a.bu != nullptr ? a.bu[n] : 0.0f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t tok = tok0 + 4 * kg + v;
                if (tok < rows) {
                    const float gv = g[v] > 0.0f ? g[v] : 0.0f;
                    const float uv = u[v] + bu;
                    a.h[tok * ffn + n] = gv > 0.0f && uv > 0.0f ? __fmul_rn(gv, uv) : 0.0f;
                }
            }
        }
    }
}

// Nonzero entries of each row of h, ascending (Turbo Sparse summary, per-layer
// zero-activation figure: only the active neurons enter W_down).
__global__ __launch_bounds__(256) void nonzero_lists_kernel(const float* __restrict__ h, int64_t n,
                                                            int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ cnt) {
    __shared__ uint32_t s_cnt[2][4];
    const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* hr = h + (int64_t)r * n;
    uint32_t run = 0;
    int buf = 0;
    for (int64_t base = 0; base < n; base += 256) {
        const int64_t j = base + tid;
        const bool nz = j < n && hr[j] != 0.0f;
        const uint64_t b = __ballot(nz);
        if (lane == 0) s_cnt[buf][wave] = (uint32_t)__popcll(b);
        __syncthreads();
        uint32_t before = run, total = run;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if (w < wave) before += s_cnt[buf][w];
            total += s_cnt[buf][w];
        }
        if (nz && idx != nullptr) idx[(int64_t)r * n + before + popc_below(b)] = (int32_t)j;
        run = total;
        buf ^= 1;
    }
    if (tid == 0 && cnt != nullptr) cnt[r] = (int32_t)run;
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_gemm_cfg(const MfmaArgs& a, hipStream_t stream) {
    const int tiles_m = (int)((a.m + BM - 1) / BM), tiles_n = (int)((a.n + BN - 1) / BN);
    gemm_nt_bf16_kernel<BM, BN, WM, WN><<<dim3(tiles_m * tiles_n), dim3(64 * WM * WN), 0, stream>>>(
        a.x, a.w, a.y, (int)a.m, (int)a.n, (int)a.k, a.y_bf16, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_masked_gemm(const MfmaArgs& a, hipStream_t stream) {
    if (a.m <= 0 || a.n <= 0) return hipSuccess;
    // Pick the tile width that leaves the fewest idle workgroup slots on 256 CUs.
    const int64_t tm = (a.m + 255) / 256;
    const int64_t t256 = tm * ((a.n + 255) / 256), t192 = tm * ((a.n + 191) / 192);
    auto waste = [](int64_t t) { int64_t r = (t + 255) / 256 * 256; return (double)(r - t) / r; };
    if (waste(t192) + 1e-9 < waste(t256)) return launch_gemm_cfg<256, 192, 2, 3>(a, stream);
    return launch_gemm_cfg<256, 256, 2, 4>(a, stream);
}

hipError_t launch_drelu_gate_up(const DreluArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)((a.ffn + 15) / 16);
    drelu_gate_up_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_nonzero_lists(const float* h, int64_t rows, int64_t n, int32_t* idx,
                                int32_t* cnt, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    nonzero_lists_kernel<<<dim3((unsigned)rows), dim3(256), 0, stream>>>(h, n, idx, cnt);
    return hipGetLastError();
}

}  // namespace qs
