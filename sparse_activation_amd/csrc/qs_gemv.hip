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
//   * eight lanes stream one selected W^T row segment of 128 bytes with
//     16-byte loads (eight rows per wavefront instruction), several rows in
//     flight per lane in two ping-pong register stages, and accumulate into
//     fp32 registers;
//   * the row slots of the workgroup are summed in LDS in a fixed order;
//     then either (accumulate form, fp32 outputs) the partial tile is added
//     into y, which an earlier launch cleared, with float atomics, so the
//     rounding depends on the order in which the splits arrive; or (fixed
//     order) the split's partial tile goes to the workspace and the last
//     workgroup of each column tile (device-scope counter) sums the splits
//     in split order, applies the epilogue and stores y: bitwise
//     reproducible.
//
// The ternary x int8 variant does the same with 2-bit packed weights and
// exact int32 accumulation.
#include "qs_internal.h"
#include "qs_rowsel.h"

namespace qs {
namespace {

constexpr int kNT = 256;     // threads per workgroup
constexpr int kLPR = 32;     // lanes per weight-row segment (ternary kernel)
constexpr int kRPI = 64 / kLPR;
constexpr int kNSlot = 4 * kRPI;
constexpr int kUnroll = 4;       // rows per pipeline stage per lane (ternary kernel)
constexpr int kMaxUnroll = 8;    // the fp kernel uses 8 for small token tiles
// The fp gather kernel reads 128-byte row segments: 8 lanes of 16 bytes per
// row, 8 rows per wavefront load, 32 row slots per workgroup.
constexpr int kFLPR = 8;
constexpr int kFNSlot = 4 * (64 / kFLPR);
constexpr int kFMaxCand = 2048;  // candidate rows per split (coefficients staged in LDS)

// Workgroups the split-K plan aims for: 2.5 per CU, measured best on the
// Llama-7B FFN decode gathers (12.2 us per launch against 12.6 at 768 and
// 13.0 at 512).
constexpr int kGemvTargetWG = 640;

__device__ __forceinline__ uint32_t popc_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Split-K handoff between workgroups that may sit on different XCDs (each
// with its own L2).  Every value that crosses workgroups is itself an
// agent-scope atomic access: the partials are written and read with relaxed
// agent-scope atomic stores and loads (sc1: they bypass the XCD's
// non-coherent L2, so each is coherent across the device on its own), and the
// counter is a relaxed agent-scope RMW.  What orders a workgroup's partial
// stores before its counter increment is the hardware wait for their
// completion: each wave waits for its own stores (s_waitcnt vmcnt(0), 0x0F70;
// an sc1 store completes at the device's coherence point), and the workgroup
// barrier orders all waves before thread 0's increment.  An acquire-release
// RMW would express the same order in the language's memory model, but at
// agent scope it writes back and invalidates the whole L2 of the XCD
// (buffer_wbl2 / buffer_inv) in every workgroup: a 16-token FFN step in the
// fixed-order mode measured 111 us with it; the protocol relies on this
// gfx950 behaviour of sc1 accesses instead.
template <typename T>
__device__ __forceinline__ void store_agent(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T load_agent(const T* p) {
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Returns true in every thread of the last workgroup to finish its split.
__device__ __forceinline__ bool last_split_arrived(int32_t* counter, int nsplit, int* s_flag) {
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0)
        *s_flag = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == nsplit - 1;
    __syncthreads();
    return *s_flag != 0;
}

// Raw buffer view of a weight matrix: out-of-range offsets read as zero.
// Weight matrices are below 1 GiB (checked by the host), so an offset with
// either part set to kOOB is out of range, and the sum cannot wrap.
constexpr uint32_t kOOB = 0x40000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const void* p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

template <int WBF16>
__device__ __forceinline__ void unpack(const u32x4& v, float* w) {
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
    } else if (a.epilogue == EPI_RELU2_GLU) {
        const float g = a.gate[i];
        reinterpret_cast<float*>(a.y)[i] = g > 0.0f ? __fmul_rn(__fmul_rn(g, g), s) : 0.0f;
    } else if (a.y_bf16) {
        reinterpret_cast<uint16_t*>(a.y)[i] = f32_to_bf16_rne(s);
    } else {
        reinterpret_cast<float*>(a.y)[i] = s;
    }
}

// Gated squared ReLU of a (gate, up) pair of sums: relu(g)^2 * u.
__device__ __forceinline__ float relu2_glu(float g, float u) {
    return g > 0.0f ? __fmul_rn(__fmul_rn(g, g), u) : 0.0f;
}

// Inclusive prefix sum over a wavefront (DPP row shifts and broadcasts).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// DUAL: a second matrix (a.w2, the gate) is streamed at the same rows into a
// second set of sums, and the output is relu2_glu(gate, up).
// With a.sel_desc, xs is not yet sparsified: each token's coefficients are
// kept only where the top-k descriptor (tau, cutoff) of its row selects them
// (Turbo Sparse summary, Eq. 3-4: the top-k% of the intermediate by |h|
// before W_down), so no selection launch and no sparsified copy are needed.
template <int WBF16, int BT, bool DUAL = false>
__global__ __launch_bounds__(kNT) void gather_gemv_kernel(GemvArgs a, int cand, int nsplit) {
    constexpr int EPT = WBF16 ? 8 : 4;
    constexpr int CT = kFLPR * EPT;                      // 128-byte row segments
    constexpr int TG = BT < 2 ? BT : 2;
    // rows per stage per lane (the dual kernel keeps the same bytes in flight)
    constexpr int U = (BT <= 4 && !DUAL) ? kMaxUnroll : kUnroll;
    constexpr int BATCH = kFNSlot * U;                   // rows per pipeline stage
    constexpr int MAXC = 8192 / BT < kFMaxCand ? 8192 / BT : kFMaxCand;   // as in the plan
    constexpr int NCH = MAXC / kNT;                                      // candidate chunks
    extern __shared__ float smem[];
    float* s_coef = smem;                                  // [cand + 3 BATCH][BT]
    uint32_t* s_off = reinterpret_cast<uint32_t*>(smem + (size_t)(cand + 3 * BATCH) * BT);
    __shared__ int s_wcnt[4];
    __shared__ int s_last;

    const int tile = blockIdx.x, split = blockIdx.y, tt = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t rows = a.rows, d_in = a.d_in, n_out = a.n_out;
    const int64_t j0 = (int64_t)split * cand;
    const int64_t j1 = min(d_in, j0 + (int64_t)cand);
    const int64_t tok0 = (int64_t)tt * BT;

    const int64_t esize = WBF16 ? 2 : 4;
    const uint32_t rowbytes = (uint32_t)((a.w_ld > 0 ? a.w_ld : n_out) * esize);   // row pitch

    // Phase A: rows of [j0, j1) selected by any token of the tile.  All the
    // coefficient loads are issued at once (candidate j0 + ch * 256 + tid is
    // chunk ch of thread tid; rows past the range or the batch read 0), one
    // block scan of the per-thread counts places them, in (thread, chunk)
    // order: s_off holds their byte offsets in W^T, s_coef their coefficients.
    const int64_t ntok = min((int64_t)BT, rows - tok0);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.xs + tok0 * d_in), (short)0, (int)(ntok * d_in * 4), 0x00020000);
    float c[NCH][BT];
    uint32_t selbits = 0;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const int64_t j = j0 + ch * kNT + tid;
        const bool jin = j < j1;
#pragma unroll
        for (int t = 0; t < BT; ++t)
            c[ch][t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                xr, jin ? (uint32_t)((t * d_in + j) * 4) : kOOB, 0, 0));
    }
    auto apply_desc = [&](int t, uint32_t tau, uint32_t cut) {
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            const uint32_t j = (uint32_t)(j0 + ch * kNT + tid);
            if (!rowsel::selected(__float_as_uint(c[ch][t]) & 0x7FFFFFFFu, j, tau, cut))
                c[ch][t] = 0.0f;
        }
    };
    if (a.sel_desc != nullptr) {   // uniform
#pragma unroll
        for (int t = 0; t < BT; ++t) {
            if (t >= ntok) break;   // uniform
            apply_desc(t, a.sel_desc[tok0 + t], a.sel_desc[rows + tok0 + t]);
        }
    }
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        bool any = false;
#pragma unroll
        for (int t = 0; t < BT; ++t) any = any || (c[ch][t] != 0.0f);
        selbits |= (any ? 1u : 0u) << ch;
    }
    const uint32_t mycnt = (uint32_t)__popc(selbits);
    const uint32_t incl = wave_incl_scan_u32(mycnt);
    if (lane == 63) s_wcnt[wave] = (int)incl;
    __syncthreads();
    int before = 0, nact = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int cw = s_wcnt[w];
        if (w < wave) before += cw;
        nact += cw;
    }
    int pos = before + (int)(incl - mycnt);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        if (selbits & (1u << ch)) {
            s_off[pos] = (uint32_t)(j0 + ch * kNT + tid) * rowbytes;
#pragma unroll
            for (int t = 0; t < BT; ++t) s_coef[pos * BT + t] = c[ch][t];
            ++pos;
        }
    }
    // Pad the list with rows that read as zero up to an even number of
    // pipeline stages plus the one stage that the last iteration prefetches.
    const int nbatch = (nact + BATCH - 1) / BATCH;
    const int npad = ((nbatch + 1) / 2 * 2 + 1) * BATCH;
    for (int i = nact + tid; i < npad; i += kNT) {
        s_off[i] = kOOB;
#pragma unroll
        for (int t = 0; t < BT; ++t) s_coef[i * BT + t] = 0.0f;
    }
    __syncthreads();

    // Phase B: stream the selected W^T row segments, one stage ahead.
    const int slot = wave * (64 / kFLPR) + lane / kFLPR;
    const int64_t col = (int64_t)tile * CT + (lane % kFLPR) * EPT;
    const uint32_t colb = col < n_out ? (uint32_t)(col * esize) : kOOB;
    const void* wbase = a.w;
    if (BT == 1 && a.row_expert != nullptr)
        wbase = reinterpret_cast<const char*>(a.w) + (int64_t)a.row_expert[tok0] * a.expert_bytes;
    const __amdgpu_buffer_rsrc_t rs = weight_rsrc(wbase, a.d_in * (int64_t)rowbytes);
    const __amdgpu_buffer_rsrc_t rs2 = weight_rsrc(DUAL ? a.w2 : wbase, a.d_in * (int64_t)rowbytes);
    constexpr int NM = DUAL ? 2 : 1;   // matrices streamed: [0] = w, [1] = w2

    float acc[NM][BT][EPT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
            for (int e = 0; e < EPT; ++e) acc[m][t][e] = 0.0f;

    // Two register buffers in ping-pong (no copies, so the waits on one stage
    // never cover the loads of the next): 2 * U rows in flight per lane and matrix.
    u32x4 bufa[NM][U], bufb[NM][U];
    auto load_stage = [&](u32x4 (*dst)[U], int bi) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t off = s_off[bi * BATCH + slot + u * kFNSlot] + colb;
            dst[0][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
            if constexpr (DUAL) dst[NM - 1][u] = __builtin_amdgcn_raw_buffer_load_b128(rs2, off, 0, 0);
        }
    };
    auto fma_stage = [&](const u32x4 (*src)[U], int bi) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ai = bi * BATCH + slot + u * kFNSlot;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                float w[EPT];
                unpack<WBF16>(src[m][u], w);
#pragma unroll
                for (int t = 0; t < BT; ++t) {
                    const float c = s_coef[ai * BT + t];
#pragma unroll
                    for (int e = 0; e < EPT; ++e) acc[m][t][e] = fmaf(c, w[e], acc[m][t][e]);
                }
            }
        }
    };
    // Straight-line body: stages past the list hold out-of-range offsets and
    // zero coefficients, so their loads return zero without memory traffic.
    // sched_barrier keeps each stage's loads issued before the previous
    // stage's arithmetic (the scheduler would otherwise sink them).
    load_stage(bufa, 0);
    for (int bi = 0; bi < nbatch; bi += 2) {
        load_stage(bufb, bi + 1);
        __builtin_amdgcn_sched_barrier(0);
        fma_stage(bufa, bi);
        __builtin_amdgcn_sched_barrier(0);
        load_stage(bufa, bi + 2);
        __builtin_amdgcn_sched_barrier(0);
        fma_stage(bufb, bi + 1);
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();   // s_coef / s_off are dead from here: reuse as the reduction buffer

    // Phase C: sum the row slots in slot order, token group by token group
    // (and, for the dual kernel, the gate's sums first).
    float* s_red = smem;   // [kFNSlot][TG][CT]
    const int cl = (lane % kFLPR) * EPT;
    constexpr int OPT = (TG * CT + kNT - 1) / kNT;   // outputs per thread and token group
#pragma unroll
    for (int t0 = 0; t0 < BT; t0 += TG) {
        float gsum[OPT];
#pragma unroll
        for (int m = NM - 1; m >= 0; --m) {
#pragma unroll
            for (int g = 0; g < TG; ++g)
#pragma unroll
                for (int e = 0; e < EPT; ++e) s_red[(slot * TG + g) * CT + cl + e] = acc[m][t0 + g][e];
            __syncthreads();
#pragma unroll
            for (int q = 0; q < OPT; ++q) {
                const int o = q * kNT + tid;
                float s = 0.0f;
                if (o < TG * CT) {
#pragma unroll
                    for (int sl = 0; sl < kFNSlot; ++sl) s += s_red[sl * TG * CT + o];
                }
                const int64_t row = o < TG * CT ? tok0 + t0 + o / CT : rows;   // rows: no store
                const int64_t cg = (int64_t)tile * CT + (o % CT);
                if (m == 1) {   // gate (dual kernel only)
                    gsum[q] = s;
                    if (row < rows && cg < n_out) {
                        if (a.accumulate) unsafeAtomicAdd(&a.y2[row * n_out + cg], s);
                        else if (nsplit > 1) store_agent(&a.partial2[((int64_t)split * rows + row) * n_out + cg], s);
                    }
                } else if (row < rows && cg < n_out) {
                    if (a.accumulate) {
                        int64_t orow = row;
                        float v = s;
                        if (BT == 1 && a.row_out != nullptr) {
                            orow = a.row_out[row];
                            v = __fmul_rn(a.row_scale[row], s);
                        }
                        unsafeAtomicAdd(&reinterpret_cast<float*>(a.y)[orow * n_out + cg], v);
                    }
                    else if (nsplit > 1) store_agent(&a.partial[((int64_t)split * rows + row) * n_out + cg], s);
                    else if (DUAL) reinterpret_cast<float*>(a.y)[row * n_out + cg] = relu2_glu(gsum[q], s);
                    else store_final(a, row * n_out + cg, s);
                }
            }
            __syncthreads();
        }
    }

    // Phase D: the last split of this tile sums the partials in split order
    // (in the accumulate form the atomics above already formed y).
    if (nsplit > 1 && !a.accumulate) {
        const int ci = tt * gridDim.x + tile;
        if (last_split_arrived(&a.counters[ci], nsplit, &s_last)) {
            for (int o = tid; o < BT * CT; o += kNT) {
                const int64_t row = tok0 + o / CT;
                const int64_t cg = (int64_t)tile * CT + (o % CT);
                if (row < rows && cg < n_out) {
                    // 16 independent loads in flight, summed in split order.
                    const int64_t stride = rows * n_out;
                    auto split_sum = [&](const float* pp) {
                        float s = 0.0f;
                        for (int sp0 = 0; sp0 < nsplit; sp0 += 16) {
                            float v[16];
#pragma unroll
                            for (int u = 0; u < 16; ++u)
                                v[u] = sp0 + u < nsplit ? load_agent(pp + (int64_t)(sp0 + u) * stride) : 0.0f;
#pragma unroll
                            for (int u = 0; u < 16; ++u)
                                if (sp0 + u < nsplit) s += v[u];
                        }
                        return s;
                    };
                    const float s = split_sum(a.partial + row * n_out + cg);
                    if constexpr (DUAL)
                        reinterpret_cast<float*>(a.y)[row * n_out + cg] =
                            relu2_glu(split_sum(a.partial2 + row * n_out + cg), s);
                    else
                        store_final(a, row * n_out + cg, s);
                }
            }
            if (tid == 0) store_agent(&a.counters[ci], 0);
        }
    }
}

// ---------------------------------------------------------------------------
// Down projection of a one-token FFN with the selection of h inside the
// gather (Turbo Sparse summary, Eq. 3-4: the top-k% of h by |h| before
// W_down).  One workgroup of 1024 threads per CU (a 64-column tile of y and a
// split of the candidate rows): each finds the top-k descriptor of the whole
// row of h itself (rowsel::select_desc31, as the descriptor launch does),
// and every wavefront lists the entries of its own share of the split that
// the descriptor selects (ballots into its own LDS segment: no workgroup
// barrier between the search and the stream) and streams their rows of
// W_down^T: eight lanes per 128-byte row segment (eight rows per wavefront
// load), up to 8 loads per lane and stage in two ping-pong register stages,
// no loads past the list's end.  The 128 row slots are summed in a fixed
// order (one DPP rotation, then 64 rows in LDS).
// ---------------------------------------------------------------------------
constexpr int kFsNT = 1024;
constexpr int kFsU = 8;                     // loads per lane and stage
constexpr int kFsMaxCand = 4 * kFsNT;       // candidates per split
constexpr int kFsCols = kFLPR * 8;          // 64 bf16 columns per tile

// Words of the selection scratch (whole 256-byte blocks) and of the kernel's
// LDS: the scratch (which the 64 x 64 reduction rows reuse), each
// wavefront's list of row offsets and coefficients, the split flag.
template <int NQ>
__host__ __device__ constexpr int fs_sel_words() {
    return (int)((sizeof(rowsel::Sel31Lds<NQ, kFsNT / 64>) / 4 + 63) / 64 * 64);
}
template <int NQ>
__host__ __device__ constexpr int fs_lds_words() {
    return fs_sel_words<NQ>() + 2 * (kFsNT / 64) * (kFsMaxCand / kFsNT) * 64 + 1;
}
static_assert(64 * kFsCols <= fs_sel_words<1>(), "reduction rows fit in the selection scratch");

template <int NQ>
__global__ __launch_bounds__(kFsNT) void gather_sel_kernel(GemvArgs a, int cand, int nsplit) {
    constexpr int NCH = kFsMaxCand / kFsNT;
    constexpr int NW = kFsNT / 64;
    constexpr int kWCap = NCH * 64;   // a wavefront's candidates
    // All LDS is dynamic, from offset 0 (a selection scratch placed behind
    // static variables ran its search more than twice as slowly): the
    // selection scratch (later the reduction rows), then each wavefront's row
    // list, then the split flag.
    extern __shared__ __attribute__((aligned(256))) float smem[];
    constexpr int kSelWords = fs_sel_words<NQ>();
    uint32_t* s_woff = reinterpret_cast<uint32_t*>(smem + kSelWords);             // [NW][kWCap]
    float* s_wcoef = smem + kSelWords + NW * kWCap;                               // [NW][kWCap]
    int* s_last = reinterpret_cast<int*>(smem + kSelWords + 2 * NW * kWCap);

    const int tile = blockIdx.x, split = blockIdx.y;
    const int64_t row = blockIdx.z;   // (split partials: one row)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t d_in = a.d_in, n_out = a.n_out;
    const int64_t j0 = (int64_t)split * cand;
    const int64_t j1 = min(d_in, j0 + (int64_t)cand);
    const uint32_t rowbytes = (uint32_t)((a.w_ld > 0 ? a.w_ld : n_out) * 2);   // row pitch

    // The split's candidate coefficients (entry j0 + ch * 1024 + tid is chunk
    // ch of thread tid) and the whole row's keys, 4 entries per run.
    const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.xs + row * d_in), (short)0, (int)(d_in * 4), 0x00020000);
    float c[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const int64_t j = j0 + ch * kFsNT + tid;
        c[ch] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            hr, j < j1 ? (uint32_t)(j * 4) : kOOB, 0, 0));
    }
    auto& L = *reinterpret_cast<rowsel::Sel31Lds<NQ, NW>*>(smem);
    rowsel::sel31_clear<kFsNT, NQ>(L, tid);
    uint32_t key[4 * NQ];   // past the row end (d_in % 4 == 0) the loads read 0
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
            hr, (uint32_t)((q * 4 * kFsNT + 4 * tid) * 4), 0, 0);
        key[4 * q] = v.x & 0x7FFFFFFFu; key[4 * q + 1] = v.y & 0x7FFFFFFFu;
        key[4 * q + 2] = v.z & 0x7FFFFFFFu; key[4 * q + 3] = v.w & 0x7FFFFFFFu;
    }
    // (an empty asm per key: the compiler would otherwise keep the loaded
    // words as well, to recompute each key where it is used)
#pragma unroll
    for (int i = 0; i < 4 * NQ; ++i) asm volatile("" : "+v"(key[i]));
    __syncthreads();
    // Once level 1 of the search is known, the candidates whose keys lie in a
    // higher level-1 bin are selected for sure: each thread touches the
    // 128-byte line of its tile's segment of such a row (one 4-byte load), so
    // those lines come from HBM into the caches while the search finishes.
    // The search's barriers order LDS only, so these loads stay in flight.
    const __amdgpu_buffer_rsrc_t rs = weight_rsrc(a.w, d_in * (int64_t)rowbytes);
    const uint32_t tileb = (uint32_t)tile * kFsCols * 2;
    uint32_t pf = 0;
    auto prefetch = [&](uint32_t b1) {
        // one load per thread, for a row of the split's first 1024 entries
        // only (about a third of the selected rows): HBM delivers that much
        // before the stream starts; touching more rows (one per thread
        // wherever it lies) had the stream read lines whose touch was still
        // in flight a second time.  More loads per wave would stall the
        // search behind their issue.
        const int64_t j = j0 + tid;
        const uint32_t kc = __float_as_uint(c[0]) & 0x7FFFFFFFu;
        const uint32_t off = j < j1 && (kc >> 20) > b1 ? (uint32_t)j * rowbytes + tileb : kOOB;
        pf = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
    };
    uint32_t tau, cut;
    rowsel::select_desc31<kFsNT, NQ>(key, d_in, a.sel_k, L, tid, tau, cut, prefetch);

    // This wavefront's selected nonzero candidates (entries j0 + ch * 1024 +
    // 64 wave + lane) as a list in its own LDS segment, in (ch, lane) order.
    uint32_t* w_off = s_woff + wave * kWCap;
    float* w_coef = s_wcoef + wave * kWCap;
    uint32_t n = 0;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const int64_t j = j0 + ch * kFsNT + tid;
        const bool on = j < j1 && c[ch] != 0.0f &&
                        rowsel::selected(__float_as_uint(c[ch]) & 0x7FFFFFFFu, (uint32_t)j, tau, cut);
        const uint64_t m = __ballot(on);
        if (on) {
            const uint32_t p = n + sel::popc_below(m);
            w_off[p] = (uint32_t)j * rowbytes;
            w_coef[p] = c[ch];
        }
        n += (uint32_t)__popcll(m);
    }
    n = __builtin_amdgcn_readfirstlane(n);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // Stream the listed rows' 128-byte segments, one stage ahead: wavefront
    // load li covers list entries 8 li .. 8 li + 7 (lane / 8 picks the row).
    const int rsub = lane / kFLPR;
    const int64_t col = (int64_t)tile * kFsCols + (lane % kFLPR) * 8;
    const uint32_t colb = col < n_out ? (uint32_t)(col * 2) : kOOB;
    const int nld = (int)((n + kFLPR - 1) / kFLPR);
    const int nst = (nld + kFsU - 1) / kFsU;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    u32x4 bufa[kFsU], bufb[kFsU];
    auto load_stage = [&](u32x4* dst, int st) {
#pragma unroll
        for (int u = 0; u < kFsU; ++u) {
            const int li = st * kFsU + u;
            if (li < nld) {   // uniform
                const int r = li * kFLPR + rsub;
                dst[u] = __builtin_amdgcn_raw_buffer_load_b128(
                    rs, (r < (int)n ? w_off[r] : kOOB) + colb, 0, 0);
            }
        }
    };
    auto fma_stage = [&](const u32x4* src, int st) {
#pragma unroll
        for (int u = 0; u < kFsU; ++u) {
            const int li = st * kFsU + u;
            if (li < nld) {   // uniform
                const int r = li * kFLPR + rsub;
                const float cf = r < (int)n ? w_coef[r] : 0.0f;
                float w[8];
                unpack<1>(src[u], w);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = fmaf(cf, w[e], acc[e]);
            }
        }
    };
    load_stage(bufa, 0);
    load_stage(bufb, 1);
    for (int st = 0; st < nst; st += 2) {   // uniform
        __builtin_amdgcn_sched_barrier(0);
        fma_stage(bufa, st);
        __builtin_amdgcn_sched_barrier(0);
        if (st + 2 < nst) load_stage(bufa, st + 2);
        __builtin_amdgcn_sched_barrier(0);
        if (st + 1 < nst) fma_stage(bufb, st + 1);
        __builtin_amdgcn_sched_barrier(0);
        if (st + 3 < nst) load_stage(bufb, st + 3);
    }

    // (the touched lines' values are not needed: an empty asm consumes them)
    asm volatile("" : : "v"(pf));

    // Fixed-order sum of the 128 slots: slots 2r and 2r + 1 of a 16-lane row
    // by one DPP rotation, then the 64 rows in LDS in row order.
    __syncthreads();   // the list is dead: the reduction buffer overwrites it
    float* s_red = smem;   // [64][kFsCols]
    const int rrow = wave * 4 + (lane >> 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float v = acc[e];
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
        if ((lane & 15) < kFLPR) s_red[rrow * kFsCols + (lane & 15) * 8 + e] = v;
    }
    __syncthreads();
    {
        // 16 lanes per column (one 16-lane row): lane `part` sums rows 4 part
        // .. 4 part + 3, then an inclusive DPP scan across the row (row_shr 1,
        // 2, 4, 8) leaves the column's total, in a fixed order, in lane 15.
        const int col = tid >> 4, part = tid & 15;
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) s += s_red[(4 * part + i) * kFsCols + col];
        s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x111, 0xF, 0xF, true));
        s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x112, 0xF, 0xF, true));
        s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x114, 0xF, 0xF, true));
        s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x118, 0xF, 0xF, true));
        const int64_t cg = (int64_t)tile * kFsCols + col;
        if (part == 15 && cg < n_out) {
            if (a.accumulate) unsafeAtomicAdd(&reinterpret_cast<float*>(a.y)[row * n_out + cg], s);
            else if (nsplit > 1) store_agent(&a.partial[(int64_t)split * n_out + cg], s);
            else store_final(a, cg, s);
        }
    }
    // The last split of this tile sums the partials in split order.
    if (nsplit > 1 && !a.accumulate) {
        if (last_split_arrived(&a.counters[tile], nsplit, s_last)) {
            if (tid < kFsCols) {
                const int64_t cg = (int64_t)tile * kFsCols + tid;
                if (cg < n_out) {
                    float s = 0.0f;
                    for (int sp = 0; sp < nsplit; ++sp) s += load_agent(&a.partial[(int64_t)sp * n_out + cg]);
                    store_final(a, cg, s);
                }
            }
            if (tid == 0) store_agent(&a.counters[tile], 0);
        }
    }
}

// ---------------------------------------------------------------------------
// Up projection of a small-batch squared-ReLU FFN without a K split (Q-Sparse
// news article, section "Sparsification with the Top-K function": X (.) M
// replaces X in the product, so only the rows of W_up^T that some token
// selects are read).
//
//   * each workgroup (512 threads) finds the top-k of each token's bf16 x
//     itself (two LDS histogram levels over the 15-bit magnitude keys, see
//     rowsel::select15_masks), so no selection launch precedes it;
//   * it owns a tile of 64 output columns over ALL rows that some token of
//     its tile selects: every wavefront lists the selected entries of its own
//     run of the row (a wavefront scan into its own LDS segment, no
//     workgroup barrier) with their coefficients, then eight lanes stream one
//     128-byte row segment with 16-byte loads (eight rows per wavefront load),
//     up to U loads per lane and stage in two ping-pong register stages, none
//     past the list's end, fp32 FMA;
//   * the 64 row slots are summed with one DPP rotation and then in LDS, in a
//     fixed order, so u is complete (no split partials, no atomics, bitwise
//     reproducible) and the activation is applied here: h = relu(u)^2, or
//     with the gate (DUAL) h = relu(g)^2 * u;
// ---------------------------------------------------------------------------
constexpr int kUcNT = 512;                   // threads per workgroup
constexpr int kUcLPR = 8;                    // lanes per 128-byte row segment
constexpr int kUcSlots = kUcNT / kUcLPR;     // 64 row slots per workgroup
constexpr int kUcCols = kUcLPR * 8;          // 64 bf16 columns per tile
constexpr int kUcPf = 1;                     // lines warmed per thread during the selection (more stall it)

// Rows per lane and pipeline stage: one token streams 16 (a Llama-7B
// selection in two stages), more tokens or the gated pair 8.  (1024 threads
// with 8 rows each streamed as fast but selected more slowly.)
template <int BT, bool DUAL>
constexpr int uc_unroll() { return BT == 1 && !DUAL ? 16 : 8; }

// Entries of the padded workgroup-wide row list for rows of length d (the
// stage loop reads one stage past an even number of stages).
constexpr int64_t uc_list_cap(int64_t d, int u) {
    const int64_t batch = (int64_t)kUcSlots * u;
    const int64_t nb = (d + batch - 1) / batch;
    return ((nb + 1) / 2 * 2 + 1) * batch;
}

// Words of LDS of the workgroup-wide list form before its scan totals: the
// largest of the row list, the selection scratch and the reduction rows.
template <int BT, bool DUAL>
__host__ __device__ constexpr int64_t uc_lds_tail(int64_t d) {
    const int64_t list = uc_list_cap(d, uc_unroll<BT, DUAL>()) * (1 + BT);
    const int64_t selw = (int64_t)sizeof(rowsel::Sel15Lds<BT, kUcNT / 64>) / 4;
    const int64_t red = (int64_t)(kUcNT / 16) * (DUAL ? 2 : 1) * BT * kUcCols;
    const int64_t m = list > selw ? list : selw;
    return m > red ? m : red;
}

// LDS words of the per-wavefront list form: the selection scratch (whole
// 256-byte blocks), then each wavefront's row list (64 E entries: a row
// offset and BT coefficients each); the reduction rows reuse the front once
// the stream is done.
template <int BT>
__host__ __device__ constexpr int64_t uc_sel_words() {
    return ((int64_t)sizeof(rowsel::Sel15Lds<BT, kUcNT / 64>) / 4 + 63) / 64 * 64;
}
template <int BT, int E, bool DUAL>
__host__ __device__ constexpr int64_t uc_lds_words() {
    const int64_t lists = uc_sel_words<BT>() + (int64_t)(kUcNT / 64) * 64 * E * (1 + BT);
    const int64_t red = (int64_t)(kUcNT / 16) * (DUAL ? 2 : 1) * BT * kUcCols;
    return lists > red ? lists : red;
}

template <int BT, int E, bool DUAL>
__global__ __launch_bounds__(kUcNT) void up_cols_kernel(UpColsArgs a) {
    constexpr int U = uc_unroll<BT, DUAL>();
    constexpr int NM = DUAL ? 2 : 1;
    // One token of the plain squared-ReLU form (or the linear): every
    // wavefront lists and streams its own rows.  Several tokens or the
    // gated pair: one workgroup-wide row list, streamed by all 64 row slots
    // in whole stages (measured faster for their longer lists).
    constexpr bool kWaveLists = BT == 1 && !DUAL;
    constexpr int NW = kUcNT / 64;
    // All LDS is dynamic, from offset 0 (tables behind static variables ran
    // markedly slower): the selection scratch or the row list, later the
    // reduction rows; the scan totals sit behind the largest of them.
    extern __shared__ __attribute__((aligned(256))) float smem[];

    const int tile = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t d = a.d, ffn = a.ffn;
    const int64_t tok0 = (int64_t)blockIdx.y * BT;
    const int64_t ntok = min((int64_t)BT, a.rows - tok0);

    // Side jobs for the down projection that follows: clear a slice of the
    // buffer it adds into (workgroups in turn), and its split counters.
    if (a.zero != nullptr && blockIdx.y == 0) {
        const int64_t per = (a.n_zero / 4 + gridDim.x - 1) / gridDim.x;
        for (int64_t i = tile * per + tid; i < min((tile + 1) * per, a.n_zero / 4); i += kUcNT)
            reinterpret_cast<uint4*>(a.zero)[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (a.zero_i != nullptr && tile == 0 && blockIdx.y == 0)
        for (int i = tid; i < a.n_zero_i; i += kUcNT) a.zero_i[i] = 0;

    // Phase 1: this thread's run of E entries of each token's activations
    // and the token's selection as a bit mask over the run: either from the
    // sparsified x of a selection launch (a.xs), or (a.x) the top-k of each
    // token's bf16 x found inside this workgroup (Q-Sparse news article,
    // Top-K section: the K entries of largest |x|, ties to the lower index),
    // so that no selection launch precedes this one.
    uint32_t selm[BT];
    float xv[BT][E];
    const int nvalid = (int)d - tid * E;
    const uint32_t rowbytes = (uint32_t)((a.w_ld > 0 ? a.w_ld : ffn) * 2);   // row pitch
    const __amdgpu_buffer_rsrc_t rs = weight_rsrc(a.w, d * (int64_t)rowbytes);
    const __amdgpu_buffer_rsrc_t rs2 = weight_rsrc(DUAL ? a.w2 : a.w, d * (int64_t)rowbytes);
    uint32_t pf[NM][kUcPf];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int g = 0; g < kUcPf; ++g) pf[m][g] = 0;
    if (a.xs != nullptr) {   // uniform
#pragma unroll
        for (int t = 0; t < BT; ++t) {
            const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(a.xs + (tok0 + t) * d), (short)0,
                t < ntok ? (int)(d * 4) : 0, 0x00020000);
#pragma unroll
            for (int q = 0; q < E / 4; ++q) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
                    xr, (uint32_t)((tid * E + 4 * q) * 4), 0, 0);
                xv[t][4 * q] = __uint_as_float(v.x); xv[t][4 * q + 1] = __uint_as_float(v.y);
                xv[t][4 * q + 2] = __uint_as_float(v.z); xv[t][4 * q + 3] = __uint_as_float(v.w);
            }
        }
#pragma unroll
        for (int t = 0; t < BT; ++t) {
            selm[t] = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) selm[t] |= (xv[t][e] != 0.0f ? 1u : 0u) << e;
        }
    } else {
        auto& L = *reinterpret_cast<rowsel::Sel15Lds<BT, NW>*>(smem);
        uint32_t xr16[BT][E / 2];   // bf16 pairs
#pragma unroll
        for (int t = 0; t < BT; ++t) {
            const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(a.x + (tok0 + t) * d), (short)0,
                t < ntok ? (int)(d * 2) : 0, 0x00020000);
#pragma unroll
            for (int q = 0; q < E / 8; ++q) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
                    xr, (uint32_t)((tid * E + 8 * q) * 2), 0, 0);
                xr16[t][4 * q] = v.x; xr16[t][4 * q + 1] = v.y; xr16[t][4 * q + 2] = v.z; xr16[t][4 * q + 3] = v.w;
            }
        }
        for (int i = tid; i < (int)(sizeof(L) / 4); i += kUcNT) reinterpret_cast<uint32_t*>(&L)[i] = 0;
        uint32_t key[BT][E];
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
            for (int e = 0; e < E; ++e)
                key[t][e] = e < nvalid ? (xr16[t][e / 2] >> (16 * (e % 2))) & 0x7FFFu : sel::kInvalid;
        // One token keeping at least a quarter of x: each thread's largest
        // |x| is selected unless all its E entries fall below the cut, which
        // for independent entries has probability at most (3/4)^E, so its
        // row's line is touched at once (before the search, about 1.2 us
        // earlier than at level 1).
        const bool early = BT == 1 && (int64_t)4 * a.k >= d;   // uniform
        if (early) {
            uint32_t bk = 0, off = kOOB;
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (key[0][e] != sel::kInvalid && key[0][e] > bk) {
                    bk = key[0][e];
                    off = (uint32_t)(tid * E + e) * rowbytes + (uint32_t)tile * kUcCols * 2;
                }
            pf[0][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
            if constexpr (DUAL) pf[1][0] = __builtin_amdgcn_raw_buffer_load_b32(rs2, off, 0, 0);
        }
        __syncthreads();
        // Once level 1 of the search is known, the entries whose keys lie in
        // a higher level-1 bin are selected for sure: each thread touches the
        // 128-byte line of this tile's segment of up to kUcPf such rows (one
        // 4-byte load each, the first such entry of each group of E / kUcPf),
        // so those lines come from HBM into the caches while the search
        // finishes.  The barriers up to the stream order LDS only, so these
        // loads stay in flight.
        const uint32_t tileb = (uint32_t)tile * kUcCols * 2;
        auto prefetch = [&](int t, uint32_t b1) {
            if (t != 0 || early) return;
#pragma unroll
            for (int g = 0; g < kUcPf; ++g) {
                uint32_t off = kOOB;
#pragma unroll
                for (int e = (g + 1) * (E / kUcPf) - 1; e >= g * (E / kUcPf); --e)
                    if (key[0][e] != sel::kInvalid && (key[0][e] >> 7) > b1)
                        off = (uint32_t)(tid * E + e) * rowbytes + tileb;
                pf[0][g] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
                if constexpr (DUAL) pf[1][g] = __builtin_amdgcn_raw_buffer_load_b32(rs2, off, 0, 0);
            }
        };
        rowsel::select15_masks<kUcNT, BT, E>(key, (int)ntok, a.k, L, tid, selm, prefetch);
        if constexpr (!kWaveLists) rowsel::lds_barrier();   // the selection scratch becomes the row list
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
            for (int e = 0; e < E; ++e)
                xv[t][e] = (selm[t] >> e) & 1u ? __uint_as_float((xr16[t][e / 2] >> (16 * (e % 2))) << 16) : 0.0f;
    }

    float acc[NM][BT][8];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[m][t][e] = 0.0f;
    if constexpr (kWaveLists) {
        // Phase 2: the union of the selections over this wavefront's run of the
        // row (entries 64 E wave .. 64 E wave + 64 E - 1) as an ascending row list
        // in its own LDS segment, with each token's coefficient (0 where the
        // token does not select the row).
        constexpr int kWCap = 64 * E;
        uint32_t* w_off = reinterpret_cast<uint32_t*>(smem + uc_sel_words<BT>()) + wave * kWCap;
        float* w_coef = smem + uc_sel_words<BT>() + NW * kWCap + wave * kWCap * BT;
        uint32_t um = 0;
    #pragma unroll
        for (int t = 0; t < BT; ++t) um |= selm[t];
        const uint32_t ucnt = (uint32_t)__popc(um);
        const uint32_t uincl = sel::wave_incl_scan_dpp(ucnt);
        const int n = __builtin_amdgcn_readlane((int)uincl, 63);
        uint32_t pos = uincl - ucnt;
    #pragma unroll
        for (int e = 0; e < E; ++e) {
            if (um & (1u << e)) {
                w_off[pos] = (uint32_t)(tid * E + e) * rowbytes;
    #pragma unroll
                for (int t = 0; t < BT; ++t) w_coef[pos * BT + t] = xv[t][e];
                ++pos;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // Phase 3: stream the 128-byte segments of the listed rows, one stage
        // ahead: wavefront load li covers list entries 8 li .. 8 li + 7 (lane / 8
        // picks the row).
        const int rsub = lane / kUcLPR;
        const int64_t col = (int64_t)tile * kUcCols + (lane % kUcLPR) * 8;
        const uint32_t colb = col < ffn ? (uint32_t)(col * 2) : kOOB;
        const int nld = (n + kUcLPR - 1) / kUcLPR;
        const int nst = (nld + U - 1) / U;
        u32x4 bufa[NM][U], bufb[NM][U];
        auto load_stage = [&](u32x4 (*dst)[U], int st) {
    #pragma unroll
            for (int u = 0; u < U; ++u) {
                const int li = st * U + u;
                if (li < nld) {   // uniform
                    const int r = li * kUcLPR + rsub;
                    const uint32_t off = (r < n ? w_off[r] : kOOB) + colb;
                    dst[0][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
                    if constexpr (DUAL) dst[1][u] = __builtin_amdgcn_raw_buffer_load_b128(rs2, off, 0, 0);
                }
            }
        };
        auto fma_stage = [&](const u32x4 (*src)[U], int st) {
    #pragma unroll
            for (int u = 0; u < U; ++u) {
                const int li = st * U + u;
                if (li < nld) {   // uniform
                    const int r = li * kUcLPR + rsub;
                    float cf[BT];
    #pragma unroll
                    for (int t = 0; t < BT; ++t) cf[t] = r < n ? w_coef[r * BT + t] : 0.0f;
    #pragma unroll
                    for (int m = 0; m < NM; ++m) {
                        float w[8];
                        unpack<1>(src[m][u], w);
    #pragma unroll
                        for (int t = 0; t < BT; ++t)
    #pragma unroll
                            for (int e = 0; e < 8; ++e) acc[m][t][e] = fmaf(cf[t], w[e], acc[m][t][e]);
                    }
                }
            }
        };
        load_stage(bufa, 0);
        load_stage(bufb, 1);
        for (int st = 0; st < nst; st += 2) {   // uniform
            __builtin_amdgcn_sched_barrier(0);
            fma_stage(bufa, st);
            __builtin_amdgcn_sched_barrier(0);
            if (st + 2 < nst) load_stage(bufa, st + 2);
            __builtin_amdgcn_sched_barrier(0);
            if (st + 1 < nst) fma_stage(bufb, st + 1);
            __builtin_amdgcn_sched_barrier(0);
            if (st + 3 < nst) load_stage(bufb, st + 3);
        }
    } else {
        // Phase 2: the union of the selections as an ascending row list with each
        // token's coefficient (0 where the token does not select the row).
        constexpr int BATCH = kUcSlots * U;
        uint32_t* s_wsum = reinterpret_cast<uint32_t*>(smem + uc_lds_tail<BT, DUAL>(a.d));   // [16]
        const int64_t cap = uc_list_cap(d, U);
        uint32_t* s_off = reinterpret_cast<uint32_t*>(smem);
        float* s_coef = smem + cap;
        uint32_t um = 0;
    #pragma unroll
        for (int t = 0; t < BT; ++t) um |= selm[t];
        uint32_t nsel;
        uint32_t pos = rowsel::block_excl_scan<kUcNT, true>((uint32_t)__popc(um), s_wsum, tid, nsel);
    #pragma unroll
        for (int e = 0; e < E; ++e) {
            if (um & (1u << e)) {
                s_off[pos] = (uint32_t)(tid * E + e) * rowbytes;
    #pragma unroll
                for (int t = 0; t < BT; ++t) s_coef[pos * BT + t] = xv[t][e];   // 0 off the token's selection
                ++pos;
            }
        }
        const int nbatch = (int)((nsel + BATCH - 1) / BATCH);
        const int npad = ((nbatch + 1) / 2 * 2 + 1) * BATCH;
        for (int i = (int)nsel + tid; i < npad; i += kUcNT) {
            s_off[i] = kOOB;
    #pragma unroll
            for (int t = 0; t < BT; ++t) s_coef[i * BT + t] = 0.0f;
        }
        rowsel::lds_barrier();

        // Phase 3: stream the 128-byte segments of the selected rows.
        const int slot = tid / kUcLPR;
        const int64_t col = (int64_t)tile * kUcCols + (lane % kUcLPR) * 8;
        const uint32_t colb = col < ffn ? (uint32_t)(col * 2) : kOOB;
        u32x4 bufa[NM][U], bufb[NM][U];
        auto load_stage = [&](u32x4 (*dst)[U], int bi) {
    #pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t off = s_off[bi * BATCH + u * kUcSlots + slot] + colb;
                dst[0][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
                if constexpr (DUAL) dst[1][u] = __builtin_amdgcn_raw_buffer_load_b128(rs2, off, 0, 0);
            }
        };
        auto fma_stage = [&](const u32x4 (*src)[U], int bi) {
    #pragma unroll
            for (int u = 0; u < U; ++u) {
                const int ai = bi * BATCH + u * kUcSlots + slot;
                float cf[BT];
    #pragma unroll
                for (int t = 0; t < BT; ++t) cf[t] = s_coef[ai * BT + t];
    #pragma unroll
                for (int m = 0; m < NM; ++m) {
                    float w[8];
                    unpack<1>(src[m][u], w);
    #pragma unroll
                    for (int t = 0; t < BT; ++t)
    #pragma unroll
                        for (int e = 0; e < 8; ++e) acc[m][t][e] = fmaf(cf[t], w[e], acc[m][t][e]);
                }
            }
        };
        load_stage(bufa, 0);
        for (int bi = 0; bi < nbatch; bi += 2) {
            load_stage(bufb, bi + 1);
            __builtin_amdgcn_sched_barrier(0);
            fma_stage(bufa, bi);
            __builtin_amdgcn_sched_barrier(0);
            load_stage(bufa, bi + 2);
            __builtin_amdgcn_sched_barrier(0);
            fma_stage(bufb, bi + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // (the touched lines' values are not needed: an empty asm consumes them)
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int g = 0; g < kUcPf; ++g) asm volatile("" : : "v"(pf[m][g]));

    // Phase 4: sum the 64 row slots in a fixed order.  Inside each 16-lane
    // row the two slots of a column group are summed by one DPP rotation
    // (row_ror 8); lanes 0..7 of each row then hold the row's sums, and the
    // 32 rows of the workgroup are summed in LDS in row order (over the dead
    // row list).
    __syncthreads();
    float* s_red = smem;   // [32][NM][BT][kUcCols]
    const int rrow = wave * 4 + (lane >> 4);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = acc[m][t][e];
                v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
                if ((lane & 15) < kUcLPR)
                    s_red[((rrow * NM + m) * BT + t) * kUcCols + (lane & 15) * 8 + e] = v;
            }
    __syncthreads();
    static_assert(BT * kUcCols <= kUcNT, "one output per thread");
    if (tid < BT * kUcCols) {   // wavefront t holds token t's 64 columns
        const int t = tid / kUcCols, c = tid % kUcCols;
        float sum[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            float v = 0.0f;
#pragma unroll
            for (int r = 0; r < 4 * NW; ++r) v += s_red[((r * NM + m) * BT + t) * kUcCols + c];
            sum[m] = v;
        }
        const int64_t cg = (int64_t)tile * kUcCols + c;
        const bool valid = t < ntok && cg < ffn;
        float hv = 0.0f;
        if constexpr (DUAL) hv = relu2_glu(sum[1], sum[0]);
        else hv = a.linear ? sum[0] : sum[0] > 0.0f ? __fmul_rn(sum[0], sum[0]) : 0.0f;
        if (valid) {
            const int64_t i = (tok0 + t) * ffn + cg;
            if (a.hb != nullptr) a.hb[i] = f32_to_bf16_rne(hv);
            else a.h[i] = hv;
            if (a.h2 != nullptr) a.h2[i] = hv;
        }
    }
}

// ---------------------------------------------------------------------------
// fp32-MFMA variant for 16-token tiles of fp32 weights (bf16 weights take the
// bf16 MFMA kernel below).  With 16 tokens the gather is a (16 x rows) .
// (rows x n_out) product, so the multiply-adds go to v_mfma_f32_16x16x4_f32:
// A = the coefficients of 16 tokens for 4 selected rows (one per lane), B =
// the 4 rows' weights.  A 16-byte load gives a lane EPT consecutive columns
// of one row; the EPT values feed EPT MFMAs whose output columns are permuted
// accordingly (MFMA e, lane column j -> column j * EPT + e), so no LDS
// transpose is needed.  The four wavefronts take different 4-row groups of
// the workgroup's selected rows for the same 16 * EPT columns and are summed
// in LDS in wave order; fp32 products and sums keep the result exact to fp32
// rounding.
// ---------------------------------------------------------------------------
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int WBF16>
__global__ __launch_bounds__(kNT) void gather_mfma_kernel(GemvArgs a, int cand, int nsplit) {
    constexpr int EPT = WBF16 ? 8 : 4;
    constexpr int CT = 16 * EPT;           // columns per workgroup (128 bf16, 64 fp32)
    constexpr int BT = 16;
    constexpr int G = 4;                   // 4-row groups per wave per stage
    constexpr int BATCH = 4 * 4 * G;       // rows per workgroup stage (4 waves)
    constexpr int OPT = BT * CT / kNT;     // outputs per thread in the reductions (8)
    extern __shared__ float smem[];
    float* s_coef = smem;                                                    // [cand + 3 BATCH][16]
    uint32_t* s_off = reinterpret_cast<uint32_t*>(smem + (size_t)(cand + 3 * BATCH) * BT);
    __shared__ int s_wcnt[4];
    __shared__ int s_last;

    const int tile = blockIdx.x, split = blockIdx.y, tt = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t rows = a.rows, d_in = a.d_in, n_out = a.n_out;
    const int64_t j0 = (int64_t)split * cand;
    const int64_t j1 = min(d_in, j0 + (int64_t)cand);
    const int64_t tok0 = (int64_t)tt * BT;
    const int64_t esize = WBF16 ? 2 : 4;
    const uint32_t rowbytes = (uint32_t)((a.w_ld > 0 ? a.w_ld : n_out) * esize);   // row pitch

    // Phase A: union of the selected rows of this candidate range (as in the
    // fp32-FMA kernel), with the 16 tokens' coefficients.
    const int64_t ntok = min((int64_t)BT, rows - tok0);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.xs + tok0 * d_in), (short)0, (int)(ntok * d_in * 4), 0x00020000);
    int nact = 0;
    for (int64_t c0 = j0; c0 < j1; c0 += kNT) {
        const int64_t j = c0 + tid;
        const bool jin = j < j1;
        float c[BT];
#pragma unroll
        for (int t = 0; t < BT; ++t)
            c[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                xr, jin ? (uint32_t)((t * d_in + j) * 4) : kOOB, 0, 0));
        bool any = false;
#pragma unroll
        for (int t = 0; t < BT; ++t) any = any || (c[t] != 0.0f);
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
            s_off[pos] = (uint32_t)j * rowbytes;
#pragma unroll
            for (int t = 0; t < BT; ++t) s_coef[pos * BT + t] = c[t];
        }
        nact = total;
        __syncthreads();
    }
    const int nbatch = (nact + BATCH - 1) / BATCH;
    const int npad = ((nbatch + 1) / 2 * 2 + 1) * BATCH;
    for (int i = nact + tid; i < npad; i += kNT) {
        s_off[i] = kOOB;
#pragma unroll
        for (int t = 0; t < BT; ++t) s_coef[i * BT + t] = 0.0f;
    }
    __syncthreads();

    // Phase B: lane (kq = lane / 16, jl = lane % 16) holds row kq of each
    // 4-row group and columns jl * EPT .. + EPT of the tile; wave w takes the
    // groups w, w + 4, w + 8, w + 12 of every 64-row stage.
    const int kq = lane >> 4, jl = lane & 15;
    const int64_t col = (int64_t)tile * CT + jl * EPT;
    const uint32_t colb = col < n_out ? (uint32_t)(col * esize) : kOOB;
    const __amdgpu_buffer_rsrc_t rs = weight_rsrc(a.w, a.d_in * (int64_t)rowbytes);

    f32x4_t acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    u32x4 wa[G], wb[G];
    float ca[G], cb[G];
    auto load_stage = [&](u32x4* w, float* c, int bi) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int ai = bi * BATCH + (g * 4 + wave) * 4 + kq;
            w[g] = __builtin_amdgcn_raw_buffer_load_b128(rs, s_off[ai] + colb, 0, 0);
            c[g] = s_coef[ai * BT + jl];
        }
    };
    auto mfma_stage = [&](const u32x4* w, const float* c) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float wf[EPT];
            unpack<WBF16>(w[g], wf);
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(c[g], wf[e], acc[e], 0, 0, 0);
        }
    };
    load_stage(wa, ca, 0);
    for (int bi = 0; bi < nbatch; bi += 2) {
        load_stage(wb, cb, bi + 1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_stage(wa, ca);
        __builtin_amdgcn_sched_barrier(0);
        load_stage(wa, ca, bi + 2);
        __builtin_amdgcn_sched_barrier(0);
        mfma_stage(wb, cb);
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();   // coefficient staging is dead: reuse LDS for the wave reduction

    // Phase C: MFMA e, register v of a lane is token 4 kq + v, column jl * EPT + e
    // of the tile.  The four waves' tiles are summed in wave order.
    float* s_red = smem;   // [4][BT][CT]
#pragma unroll
    for (int e = 0; e < EPT; ++e)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            s_red[(wave * BT + 4 * kq + v) * CT + jl * EPT + e] = acc[e][v];
    __syncthreads();
    float outv[OPT];
#pragma unroll
    for (int q = 0; q < OPT; ++q) {
        const int o = q * kNT + tid;             // output index in the BT x CT tile
        float sum = s_red[o];
#pragma unroll
        for (int w = 1; w < 4; ++w) sum += s_red[w * BT * CT + o];
        outv[q] = sum;
    }
#pragma unroll
    for (int q = 0; q < OPT; ++q) {
        const int o = q * kNT + tid;
        const int64_t row = tok0 + o / CT, cg = (int64_t)tile * CT + (o % CT);
        if (row < rows && cg < n_out) {
            if (nsplit == 1) store_final(a, row * n_out + cg, outv[q]);
            else store_agent(&a.partial[((int64_t)split * rows + row) * n_out + cg], outv[q]);
        }
    }

    // Phase D: the last workgroup of this tile sums the partials in split
    // order, with the loads of all its outputs for 8 splits in flight at once.
    if (nsplit > 1) {
        const int ci = tt * gridDim.x + tile;
        if (last_split_arrived(&a.counters[ci], nsplit, &s_last)) {
            const int64_t stride = rows * n_out;
            int64_t base[OPT];
            bool ok[OPT];
            float sum[OPT];
#pragma unroll
            for (int q = 0; q < OPT; ++q) {
                const int o = q * kNT + tid;
                const int64_t row = tok0 + o / CT, cg = (int64_t)tile * CT + (o % CT);
                ok[q] = row < rows && cg < n_out;
                base[q] = ok[q] ? row * n_out + cg : 0;
                sum[q] = 0.0f;
            }
            for (int sp0 = 0; sp0 < nsplit; sp0 += 8) {
                float v[8][OPT];
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int q = 0; q < OPT; ++q)
                        v[u][q] = (sp0 + u < nsplit && ok[q])
                                      ? load_agent(a.partial + (int64_t)(sp0 + u) * stride + base[q]) : 0.0f;
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int q = 0; q < OPT; ++q)
                        if (sp0 + u < nsplit) sum[q] += v[u][q];
            }
#pragma unroll
            for (int q = 0; q < OPT; ++q)
                if (ok[q]) store_final(a, base[q], sum[q]);
            if (tid == 0) store_agent(&a.counters[ci], 0);
        }
    }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- bf16 MFMA gather
// 16-token tiles with bf16 weights run on the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16): tokens are the M side, a group of 32 consecutive
// input rows one k-step, 16 columns the N side.  Each fp32 coefficient c is
// split as hi = bf16(c), lo = bf16(c - hi): hi + lo keeps 16 significant bits,
// the products with bf16 weights are exact in the fp32 accumulator, and lo is
// dropped when the coefficients are bf16 values (bf16 activations).
//
// A fragment kernel rewrites X (.) M once, elementwise, into the MFMA A-operand
// layout, plus one 32-bit mask per row group whose bit i says that row i of the
// group is selected by at least one of the 16 tokens.  The gather kernel issues
// the loads of unselected rows at an out-of-range buffer offset, so they move no
// memory: the bytes read are those of the union of the tokens' selections.
//
// Per token tile tt (groups_total = ceil(d_in / 32)):
//   frag[tt][g][hi|lo][64 lanes] u32x4: lane 16 q + t holds token t's
//       coefficients of rows 32 g + 8 q .. 32 g + 8 q + 7
//   mask[tt][g] u32
constexpr int kBGroup = 32;
constexpr int kBCols = 64;

struct BFrag {
    u32x4* frag;
    uint32_t* mask;
    int64_t groups;     // groups_total
};

__host__ __device__ inline size_t bfrag_bytes(int64_t d_in, int n_tok_tiles) {
    const int64_t groups = (d_in + kBGroup - 1) / kBGroup;
    const size_t masks = ((size_t)n_tok_tiles * groups * 4 + 255) / 256 * 256;
    return masks + (size_t)n_tok_tiles * groups * 2 * 64 * 16;
}

__host__ inline BFrag bfrag_carve(void* base, int64_t d_in, int n_tok_tiles) {
    const int64_t groups = (d_in + kBGroup - 1) / kBGroup;
    BFrag f;
    f.groups = groups;
    f.mask = static_cast<uint32_t*>(base);
    f.frag = reinterpret_cast<u32x4*>(static_cast<char*>(base) +
                                      ((size_t)n_tok_tiles * groups * 4 + 255) / 256 * 256);
    return f;
}

// One wave per row group: lane 16 q + t converts rows 32 g + 8 q .. + 7 of
// token t.  Grid (ceil(groups / 4), token tiles), 256 threads.
__global__ __launch_bounds__(kNT) void bfrag_kernel(const float* xs, int64_t rows, int64_t d_in,
                                                   int use_lo, BFrag bf) {
    constexpr int BT = 16;
    const int tt = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (g >= bf.groups) return;
    const int q = lane >> 4, t = lane & 15;
    const int64_t tok0 = (int64_t)tt * BT;
    const int64_t ntok = min((int64_t)BT, rows - tok0);
    const int64_t j = g * kBGroup + 8 * q;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(xs + tok0 * d_in), (short)0, (int)(ntok * d_in * 4), 0x00020000);
    const uint32_t o = t < ntok ? (uint32_t)((t * d_in + j) * 4) : kOOB;
    const u32x4 v0 = __builtin_amdgcn_raw_buffer_load_b128(xr, o, 0, 0);
    const u32x4 v1 = __builtin_amdgcn_raw_buffer_load_b128(xr, o + 16, 0, 0);
    const uint32_t u[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t hw[4], lw[4], rowbits = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float c = j + e < d_in ? __uint_as_float(u[e]) : 0.0f;
        const uint32_t hi = f32_to_bf16_rne(c);
        const uint32_t lo = f32_to_bf16_rne(c - __uint_as_float(hi << 16));
        if (e & 1) {
            hw[e >> 1] |= hi << 16;
            lw[e >> 1] |= lo << 16;
        } else {
            hw[e >> 1] = hi;
            lw[e >> 1] = lo;
        }
        // Row 8 q + e of the group is selected by some token iff one of the 16
        // lanes with this q sees a nonzero coefficient.
        const uint64_t b = __ballot(c != 0.0f);
        rowbits |= (uint32_t)((b >> (16 * 0)) & 0xFFFFu ? 1u : 0u) << (e);
        rowbits |= (uint32_t)((b >> (16 * 1)) & 0xFFFFu ? 1u : 0u) << (8 + e);
        rowbits |= (uint32_t)((b >> (16 * 2)) & 0xFFFFu ? 1u : 0u) << (16 + e);
        rowbits |= (uint32_t)((b >> (16 * 3)) & 0xFFFFu ? 1u : 0u) << (24 + e);
    }
    const size_t base = ((size_t)tt * bf.groups + g) * 128;
    bf.frag[base + lane] = (u32x4){hw[0], hw[1], hw[2], hw[3]};
    if (use_lo) bf.frag[base + 64 + lane] = (u32x4){lw[0], lw[1], lw[2], lw[3]};
    if (lane == 0) bf.mask[(size_t)tt * bf.groups + g] = rowbits;
}

// Streams rows split * cand .. + cand for a 64-column tile.  Wave w takes groups
// w, w + 4, ... of the split; per stage a lane (r8 = lane / 8, c8 = lane % 8)
// loads columns 8 c8 .. 8 c8 + 7 of rows 4 r8 .. 4 r8 + 3 of the group (whole
// 128-byte row segments), which a per-wave LDS tile turns into the k-major B
// operand.  The row mask of a group is fetched one stage ahead of its weights.
// MODE 0: packed records and row masks from bfrag_kernel.
// MODE 1 (fused): no packed records; each lane loads its 8 coefficients of a
// group two stages ahead and forms its fragments and the group's row mask
// itself, as bfrag_kernel does (the same values, so the same result).
// MODE 2: packed records written by the selection kernel, no masks: each lane
// loads its records two stages ahead and the group's row mask is formed by
// ballot over their nonzero entries.  (A value whose hi and lo parts are both
// zero multiplies to zero either way, so the skipped rows change nothing.)
// DUAL: a second matrix (a.w2, the gate) is streamed at the same rows with the
// same A fragments into a second set of sums; y = relu2_glu(gate, up).
template <int MODE, bool DUAL = false>
__global__ __launch_bounds__(kNT) void gather_bmfma_kernel(GemvArgs a, BFrag bf, int cand, int nsplit,
                                                          int use_lo) {
    constexpr int BT = 16;
    constexpr int OPT = BT * kBCols / kNT;    // outputs per thread in the reductions (4)
    constexpr int NM = DUAL ? 2 : 1;
    // 16 KB per matrix: the split-K arrival flag reuses the tiles once they are dead.
    __shared__ __attribute__((aligned(16))) uint16_t s_tr[NM * 4 * kBGroup * kBCols];

    const int tile = blockIdx.x, split = blockIdx.y, tt = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t rows = a.rows, n_out = a.n_out;
    const int64_t tok0 = (int64_t)tt * BT;
    const int64_t g0 = (int64_t)split * (cand / kBGroup);
    const int64_t gl = min((int64_t)(cand / kBGroup), bf.groups - g0);   // groups of this split
    const int nst = (int)((gl + 3) / 4);

    const __amdgpu_buffer_rsrc_t mrr = __builtin_amdgcn_make_buffer_rsrc(
        bf.mask + (size_t)tt * bf.groups + g0, (short)0, (int)(gl * 4), 0x00020000);
    const __amdgpu_buffer_rsrc_t frr = __builtin_amdgcn_make_buffer_rsrc(
        bf.frag + ((size_t)tt * bf.groups + g0) * 128, (short)0, (int)(gl * 128 * 16), 0x00020000);
    const int r8 = lane >> 3, c8 = lane & 7;
    const int kq = lane >> 4, n16 = lane & 15;
    const int64_t col = (int64_t)tile * kBCols + 8 * c8;
    const uint32_t colb = col < n_out ? (uint32_t)(col * 2) : kOOB;
    const uint32_t rowbytes = (uint32_t)((a.w_ld > 0 ? a.w_ld : n_out) * 2);   // row pitch
    const __amdgpu_buffer_rsrc_t rs = weight_rsrc(a.w, a.d_in * (int64_t)rowbytes);
    const __amdgpu_buffer_rsrc_t rs2 = weight_rsrc(DUAL ? a.w2 : a.w, a.d_in * (int64_t)rowbytes);
    // Byte offset of row 4 r8 of group 0 of the split.
    const uint32_t rowb0 = (uint32_t)((g0 * kBGroup + 4 * r8) * rowbytes);
    uint16_t* tr = s_tr + wave * kBGroup * kBCols;
    uint16_t* tr2 = s_tr + (DUAL ? 4 * kBGroup * kBCols : 0) + wave * kBGroup * kBCols;

    auto load_mask = [&](int s) {
        return __builtin_amdgcn_raw_buffer_load_b32(mrr, (uint32_t)((4 * s + wave) * 4), 0, 0);
    };
    // w[0 .. 3]: the four rows of matrix w; w[4 .. 7] (dual): the same rows of w2.
    auto load_w = [&](u32x4* w, uint32_t m, int s) {
        const uint32_t rb = rowb0 + (uint32_t)((4 * s + wave) * kBGroup) * rowbytes + colb;
        const uint32_t bits = m >> (4 * r8);
        const uint32_t o[4] = {bits & 1u ? rb : kOOB, bits & 2u ? rb + rowbytes : kOOB,
                               bits & 4u ? rb + 2 * rowbytes : kOOB, bits & 8u ? rb + 3 * rowbytes : kOOB};
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, o[q], 0, 0);
        if constexpr (DUAL) {
#pragma unroll
            for (int q = 0; q < 4; ++q) w[4 + q] = __builtin_amdgcn_raw_buffer_load_b128(rs2, o[q], 0, 0);
        }
    };
    auto load_f = [&](u32x4* f, int s) {
        const uint32_t fo = (uint32_t)(((4 * s + wave) * 128 + lane) * 16);
        f[0] = __builtin_amdgcn_raw_buffer_load_b128(frr, fo, 0, 0);
        f[1] = __builtin_amdgcn_raw_buffer_load_b128(frr, use_lo ? fo + 64 * 16 : kOOB, 0, 0);
    };
    // FUSED: lane (kq, n16) holds coefficients 8 kq .. 8 kq + 7 of the group
    // for token n16 (the A-operand layout of bfrag_kernel).
    const int64_t d_in = a.d_in;
    const int64_t ntok = min((int64_t)BT, rows - tok0);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.xs + tok0 * d_in), (short)0, (int)(ntok * d_in * 4), 0x00020000);
    auto load_x = [&](u32x4* x, int s) {
        const int64_t g = g0 + 4 * s + wave;
        const int64_t j = g * kBGroup + 8 * kq;
        if constexpr (MODE == 2) {
            // Records of tokens past the batch and of chunks past d_in were
            // never written: they load as zero.
            const uint32_t fo = (n16 < ntok && j < d_in) ? (uint32_t)(((4 * s + wave) * 128 + lane) * 16) : kOOB;
            x[0] = __builtin_amdgcn_raw_buffer_load_b128(frr, fo, 0, 0);
            x[1] = __builtin_amdgcn_raw_buffer_load_b128(frr, use_lo && fo != kOOB ? fo + 64 * 16 : kOOB, 0, 0);
            return;
        }
        const uint32_t o = (n16 < ntok && 4 * s + wave < gl) ? (uint32_t)((n16 * d_in + j) * 4) : kOOB;
        x[0] = __builtin_amdgcn_raw_buffer_load_b128(xr, o, 0, 0);
        x[1] = __builtin_amdgcn_raw_buffer_load_b128(xr, o == kOOB ? kOOB : o + 16, 0, 0);
    };
    auto convert = [&](const u32x4* x, u32x4* f, uint32_t& m, int s) {
        if constexpr (MODE == 2) {
            const uint32_t hw[4] = {x[0].x, x[0].y, x[0].z, x[0].w};
            const uint32_t lw[4] = {x[1].x, x[1].y, x[1].z, x[1].w};
            uint32_t rowbits = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t nz = ((hw[e >> 1] | lw[e >> 1]) >> (16 * (e & 1))) & 0xFFFFu;
                const uint64_t b = __ballot(nz != 0u);
                rowbits |= (uint32_t)((b & 0xFFFFull) ? 1u : 0u) << e;
                rowbits |= (uint32_t)(((b >> 16) & 0xFFFFull) ? 1u : 0u) << (8 + e);
                rowbits |= (uint32_t)(((b >> 32) & 0xFFFFull) ? 1u : 0u) << (16 + e);
                rowbits |= (uint32_t)(((b >> 48) & 0xFFFFull) ? 1u : 0u) << (24 + e);
            }
            f[0] = x[0];
            f[1] = x[1];
            m = rowbits;
            return;
        }
        const int64_t j = (g0 + 4 * s + wave) * kBGroup + 8 * kq;
        const uint32_t u[8] = {x[0].x, x[0].y, x[0].z, x[0].w, x[1].x, x[1].y, x[1].z, x[1].w};
        uint32_t hw[4], lw[4], rowbits = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float c = j + e < d_in ? __uint_as_float(u[e]) : 0.0f;
            const uint32_t hi = f32_to_bf16_rne(c);
            const uint32_t lo = f32_to_bf16_rne(c - __uint_as_float(hi << 16));
            if (e & 1) {
                hw[e >> 1] |= hi << 16;
                lw[e >> 1] |= lo << 16;
            } else {
                hw[e >> 1] = hi;
                lw[e >> 1] = lo;
            }
            const uint64_t b = __ballot(c != 0.0f);
            rowbits |= (uint32_t)((b & 0xFFFFull) ? 1u : 0u) << e;
            rowbits |= (uint32_t)(((b >> 16) & 0xFFFFull) ? 1u : 0u) << (8 + e);
            rowbits |= (uint32_t)(((b >> 32) & 0xFFFFull) ? 1u : 0u) << (16 + e);
            rowbits |= (uint32_t)(((b >> 48) & 0xFFFFull) ? 1u : 0u) << (24 + e);
        }
        f[0] = (u32x4){hw[0], hw[1], hw[2], hw[3]};
        f[1] = (u32x4){lw[0], lw[1], lw[2], lw[3]};
        m = rowbits;
    };
    f32x4_t acc[NM][4];
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mi][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    auto mfma_one = [&](const u32x4* w, uint16_t* trp, f32x4_t* ac, const u32x4* f) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = 4 * r8 + q;
            *reinterpret_cast<u32x4*>(trp + row * kBCols + ((c8 ^ (2 * (row >> 3))) * 8)) = w[q];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int cidx = ((2 * t + (n16 >> 3)) ^ (2 * kq)) * 8 + (n16 & 7);
            uint32_t bw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo16 = trp[(8 * kq + 2 * e) * kBCols + cidx];
                const uint32_t hi16 = trp[(8 * kq + 2 * e + 1) * kBCols + cidx];
                bw[e] = lo16 | (hi16 << 16);
            }
            const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, (u32x4){bw[0], bw[1], bw[2], bw[3]});
            ac[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f[0]), bv,
                                                           ac[t], 0, 0, 0);
            if (use_lo)
                ac[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f[1]),
                                                               bv, ac[t], 0, 0, 0);
        }
    };
    auto mfma_stage = [&](const u32x4* w, const u32x4* f, uint32_t m, int s) {
        if (4 * s + wave >= gl || __builtin_amdgcn_readfirstlane(m) == 0) return;
        mfma_one(w, tr, acc[0], f);
        if constexpr (DUAL) mfma_one(w + 4, tr2, acc[NM - 1], f);
    };
    // The prologue issues the loads in the loop's own order, so the wait
    // counts at the loop head are the steady-state ones.
    // The first two stages load every row without waiting for their masks
    // (a skipped row only saves bandwidth; its coefficients are zero).
    u32x4 wa[4 * NM], wb[4 * NM], fa[2], fb[2];
    if constexpr (MODE != 0) {
        // The same schedule with the coefficients (or the unmasked records)
        // in place of the records:
        // those of stage s + 2 are converted just before its weights are
        // loaded (their mask decides which rows move).
        u32x4 xa[2], xb[2], xc[2], xd[2];
        uint32_t ma, mb, mc, md;
        load_x(xa, 0);
        load_x(xb, 1);
        __builtin_amdgcn_sched_barrier(0);
        load_w(wa, 0xFFFFFFFFu, 0);
        load_x(xc, 2);
        __builtin_amdgcn_sched_barrier(0);
        load_w(wb, 0xFFFFFFFFu, 1);
        load_x(xd, 3);
        convert(xa, fa, ma, 0);
        convert(xb, fb, mb, 1);
        for (int s = 0; s < nst; s += 2) {
            __builtin_amdgcn_sched_barrier(0);
            mfma_stage(wa, fa, ma, s);
            __builtin_amdgcn_sched_barrier(0);
            convert(xc, fa, ma, s + 2);
            load_w(wa, ma, s + 2);
            load_x(xc, s + 4);
            __builtin_amdgcn_sched_barrier(0);
            mfma_stage(wb, fb, mb, s + 1);
            __builtin_amdgcn_sched_barrier(0);
            convert(xd, fb, mb, s + 3);
            load_w(wb, mb, s + 3);
            load_x(xd, s + 5);
        }
    } else {
    uint32_t ma = load_mask(0), mb = load_mask(1);
    __builtin_amdgcn_sched_barrier(0);
    load_w(wa, 0xFFFFFFFFu, 0);
    load_f(fa, 0);
    uint32_t mc = load_mask(2);
    __builtin_amdgcn_sched_barrier(0);
    load_w(wb, 0xFFFFFFFFu, 1);
    load_f(fb, 1);
    uint32_t md = load_mask(3);
    for (int s = 0; s < nst; s += 2) {
        __builtin_amdgcn_sched_barrier(0);
        mfma_stage(wa, fa, ma, s);
        __builtin_amdgcn_sched_barrier(0);
        load_w(wa, mc, s + 2);
        load_f(fa, s + 2);
        ma = mc;
        mc = load_mask(s + 4);
        __builtin_amdgcn_sched_barrier(0);
        mfma_stage(wb, fb, mb, s + 1);
        __builtin_amdgcn_sched_barrier(0);
        load_w(wb, md, s + 3);
        load_f(fb, s + 3);
        mb = md;
        md = load_mask(s + 5);
    }
    }
    __syncthreads();   // the transpose tiles are dead: reuse them for the wave reduction

    // Phase C: register v of MFMA t is token 4 kq + v, column 16 t + n16.
    float* s_red = reinterpret_cast<float*>(s_tr);   // [NM][4][16][64]
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                s_red[((mi * 4 + wave) * BT + 4 * kq + v) * kBCols + 16 * t + n16] = acc[mi][t][v];
    __syncthreads();
    float outv[NM][OPT];
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
#pragma unroll
        for (int q = 0; q < OPT; ++q) {
            const int o = q * kNT + tid;
            const float* sr = s_red + mi * 4 * BT * kBCols;
            float sum = sr[o];
#pragma unroll
            for (int w = 1; w < 4; ++w) sum += sr[w * BT * kBCols + o];
            outv[mi][q] = sum;
        }
#pragma unroll
    for (int q = 0; q < OPT; ++q) {
        const int o = q * kNT + tid;
        const int64_t row = tok0 + o / kBCols, cg = (int64_t)tile * kBCols + (o % kBCols);
        if (row < rows && cg < n_out) {
            const int64_t i = row * n_out + cg, pi = ((int64_t)split * rows + row) * n_out + cg;
            if (a.accumulate) {
                unsafeAtomicAdd(&reinterpret_cast<float*>(a.y)[i], outv[0][q]);
                if constexpr (DUAL) unsafeAtomicAdd(&a.y2[i], outv[NM - 1][q]);
            } else if constexpr (DUAL) {
                if (nsplit == 1) {
                    reinterpret_cast<float*>(a.y)[i] = relu2_glu(outv[1][q], outv[0][q]);
                } else {
                    store_agent(&a.partial[pi], outv[0][q]);
                    store_agent(&a.partial2[pi], outv[1][q]);
                }
            } else {
                if (nsplit == 1) store_final(a, i, outv[0][q]);
                else store_agent(&a.partial[pi], outv[0][q]);
            }
        }
    }

    // Phase D: the last workgroup of the tile sums the partials in split order.
    if (nsplit > 1 && !a.accumulate) {
        const int ci = tt * gridDim.x + tile;
        if (last_split_arrived(&a.counters[ci], nsplit, reinterpret_cast<int*>(s_tr))) {
            const int64_t stride = rows * n_out;
            int64_t base[OPT];
            bool ok[OPT];
            float sum[OPT];
#pragma unroll
            for (int q = 0; q < OPT; ++q) {
                const int o = q * kNT + tid;
                const int64_t row = tok0 + o / kBCols, cg = (int64_t)tile * kBCols + (o % kBCols);
                ok[q] = row < rows && cg < n_out;
                base[q] = ok[q] ? row * n_out + cg : 0;
                sum[q] = 0.0f;
            }
            auto split_sums = [&](const float* part, float* sm) {
                for (int sp0 = 0; sp0 < nsplit; sp0 += 8) {
                    float v[8][OPT];
#pragma unroll
                    for (int u = 0; u < 8; ++u)
#pragma unroll
                        for (int q = 0; q < OPT; ++q)
                            v[u][q] = (sp0 + u < nsplit && ok[q])
                                          ? load_agent(part + (int64_t)(sp0 + u) * stride + base[q]) : 0.0f;
#pragma unroll
                    for (int u = 0; u < 8; ++u)
#pragma unroll
                        for (int q = 0; q < OPT; ++q)
                            if (sp0 + u < nsplit) sm[q] += v[u][q];
                }
            };
            split_sums(a.partial, sum);
            if constexpr (DUAL) {
                float gs[OPT];
#pragma unroll
                for (int q = 0; q < OPT; ++q) gs[q] = 0.0f;
                split_sums(a.partial2, gs);
#pragma unroll
                for (int q = 0; q < OPT; ++q)
                    if (ok[q]) reinterpret_cast<float*>(a.y)[base[q]] = relu2_glu(gs[q], sum[q]);
            } else {
#pragma unroll
                for (int q = 0; q < OPT; ++q)
                    if (ok[q]) store_final(a, base[q], sum[q]);
            }
            if (tid == 0) store_agent(&a.counters[ci], 0);
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
constexpr int kI8LPR = 8;                  // lanes per row segment (64 bytes = 256 columns)
constexpr int kI8CT = kI8LPR * kI8EPT;     // 256 columns per tile
constexpr int kI8NSlot = 4 * (64 / kI8LPR);   // 32 row slots per workgroup
constexpr int kI8MaxCand = 4096;           // candidate rows per split (LDS staging)
constexpr int kI8TargetWG = 128;           // the whole matrix is a few MB: few, fuller workgroups
static_assert(kI8CT == kNT, "the slot reduction gives each thread one column");

// ---------------------------------------------------------------------------
// The quantised linear for 1-4 tokens in one launch (Q-Sparse news article,
// section "Sparsification with the Top-K function": activations quantised to
// 8 bits before the top-K; ternary weights alpha * t).  Every workgroup
//   * loads the fp32 x rows of its tokens (thread t holds entries
//     [t E, t E + E)), forms gamma = max |x| by a block reduction and q =
//     clamp(rint(x * s)), s = 127 / (gamma + 1e-5), every step IEEE binary32
//     round-to-nearest-even;
//   * finds the top-k of |q| itself: every wavefront reads the 128-bin LDS
//     histogram of the 7-bit keys from the top and finds the key tau of the
//     k-th largest and how many keys equal to it are taken; each thread then
//     ranks its own ties by a block prefix count (index order = thread order),
//     so no cutoff has to be broadcast;
//   * each thread sums q_j t_j over its own selected features for the
//     workgroup's CT output columns in exact int32 (CT / 4 packed bytes per
//     row; the loads of unselected features use an out-of-range offset and
//     move no data), then the threads' sums are added in LDS: integer sums,
//     the same in any order, so there is no K split, handoff or atomic;
//   * writes acc and y = fl32(fl32(acc) * fl32(alpha / s)); workgroup 0 also
//     writes q, s and the index list when they are asked for.
// ---------------------------------------------------------------------------
// Output columns per workgroup: 16, 4 packed bytes of each selected row
// (32 or 64 columns, with fewer cache-line requests for the same bytes, ran
// slower: the unpacking and sums per thread grow and fewer CUs take part).
constexpr int kI8Ct = 16;
// Threads per workgroup: 1024 for one token, 512 for 2-4 (the chains of
// dependent steps are per thread; 256 threads ran 5% and 9% slower).
constexpr int i8f_threads(int bt) { return bt == 1 ? 1024 : 512; }
// The |q| histogram in copies by lane (the few small |q| bins of an
// activation would serialise one copy's atomics), pitched so that a bin's
// copies sit on different LDS banks.
constexpr int kI8HistCopies = 4;
constexpr int kI8HistPitch = 128 + 16;

// One step of the wavefront butterfly below, on lane bit B, with NV >> (5 -
// B) values still held per lane (or one), then the next lower bit.
template <int NV, int B>
__device__ __forceinline__ void i8_butterfly(int32_t (&cur)[NV], int lane) {
    if constexpr (B >= 0) {
        constexpr int n = (NV >> (5 - B)) > 1 ? (NV >> (5 - B)) : 1;
        if constexpr (n > 1) {
            const bool up = (lane >> B) & 1;
#pragma unroll
            for (int i = 0; i < n / 2; ++i) {
                const int32_t send = up ? cur[i] : cur[i + n / 2];
                const int32_t keep = up ? cur[i + n / 2] : cur[i];
                cur[i] = keep + __shfl_xor(send, 1 << B);
            }
        } else {
            cur[0] += __shfl_xor(cur[0], 1 << B);
        }
        i8_butterfly<NV, B - 1>(cur, lane);
    }
}

template <int BT, int E>
__global__ __launch_bounds__(i8f_threads(BT)) void i8t_fused_kernel(I8fArgs a) {
    constexpr int NT = i8f_threads(BT);
    constexpr int CT = kI8Ct;
    constexpr int NW = NT / 64;
    __shared__ int32_t s_part[NW][BT * CT];
    __shared__ uint32_t s_wsum[16];
    __shared__ uint32_t s_tie[BT][NW];
    __shared__ float s_fmax[BT][NW];
    __shared__ uint32_t s_hist[BT][kI8HistCopies][kI8HistPitch];

    const int tile = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t d = a.d_in, n_out = a.n_out;
    const int ntok = (int)a.rows;
    const int nvalid = (int)d - tid * E;         // entries of this thread's run

    // Phase 1: x, gamma, q and the histogram of |q|.
    float xv[BT][E];
#pragma unroll
    for (int t = 0; t < BT; ++t) {
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(a.x + (int64_t)t * d), (short)0, t < ntok ? (int)(d * 4) : 0, 0x00020000);
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xr, (uint32_t)((tid * E + 4 * q) * 4), 0, 0);
            xv[t][4 * q] = __uint_as_float(v.x); xv[t][4 * q + 1] = __uint_as_float(v.y);
            xv[t][4 * q + 2] = __uint_as_float(v.z); xv[t][4 * q + 3] = __uint_as_float(v.w);
        }
    }
    for (int i = tid; i < BT * kI8HistCopies * kI8HistPitch; i += NT) (&s_hist[0][0][0])[i] = 0;
#pragma unroll
    for (int t = 0; t < BT; ++t) {
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) m = fmaxf(m, fabsf(xv[t][e]));
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        if (lane == 0) s_fmax[t][wave] = m;
    }
    __syncthreads();
    float scale[BT];
    int32_t qv[BT][E];
#pragma unroll
    for (int t = 0; t < BT; ++t) {
        float g = s_fmax[t][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) g = fmaxf(g, s_fmax[t][w]);
        scale[t] = __fdiv_rn(127.0f, __fadd_rn(g, 1e-5f));
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float r = rintf(__fmul_rn(xv[t][e], scale[t]));
            r = fminf(fmaxf(r, -128.0f), 127.0f);
            qv[t][e] = (int32_t)r;
            if (t < ntok && e < nvalid)
                atomicAdd(&s_hist[t][lane % kI8HistCopies][qv[t][e] < 0 ? -qv[t][e] : qv[t][e]], 1u);
        }
    }
    __syncthreads();

    // Phase 2: selection masks over this thread's run, per token.
    const uint32_t kk = (uint32_t)a.k;
    uint32_t selm[BT];
#pragma unroll
    for (int t = 0; t < BT; ++t) {
        selm[t] = 0;
        if (t >= ntok || kk == 0) continue;   // uniform
        // tau: lane l holds bins 127 - 2l and 126 - 2l (summed over the
        // copies); the running total from the top reaches k in exactly one lane.
        uint32_t c0 = 0, c1 = 0;
#pragma unroll
        for (int cp = 0; cp < kI8HistCopies; ++cp) {
            c0 += s_hist[t][cp][127 - 2 * lane];
            c1 += s_hist[t][cp][126 - 2 * lane];
        }
        const uint32_t incl = sel::wave_incl_scan_dpp(c0 + c1);
        const uint32_t excl = incl - c0 - c1;
        const uint64_t hit = __ballot(excl < kk && kk <= incl);
        const int src = (int)__builtin_ctzll(hit);
        const uint32_t ex = (uint32_t)__builtin_amdgcn_readlane((int)excl, src);
        const uint32_t h0 = (uint32_t)__builtin_amdgcn_readlane((int)c0, src);
        const uint32_t h1 = (uint32_t)__builtin_amdgcn_readlane((int)c1, src);
        const bool upper = kk <= ex + h0;
        const uint32_t tau = upper ? 127u - 2u * (uint32_t)src : 126u - 2u * (uint32_t)src;
        const uint32_t need = upper ? kk - ex : kk - ex - h0;   // keys equal to tau taken
        const uint32_t eqn = upper ? h0 : h1;                   // keys equal to tau in all
        uint32_t before = 0;   // keys equal to tau before this thread's run
        if (need < eqn) {      // uniform: rank the ties in index order
            uint32_t eq = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) eq += (e < nvalid && (uint32_t)abs(qv[t][e]) == tau) ? 1u : 0u;
            const uint32_t wi = sel::wave_incl_scan_dpp(eq);
            if (lane == 63) s_tie[t][wave] = wi;
            rowsel::lds_barrier();
#pragma unroll
            for (int w = 0; w < NW; ++w) before += w < wave ? s_tie[t][w] : 0u;
            before += wi - eq;
        }
        uint32_t r = before;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t kv = (uint32_t)abs(qv[t][e]);
            const bool tie = e < nvalid && kv == tau;
            const bool on = e < nvalid && (kv > tau || (tie && r < need));
            r += tie ? 1u : 0u;
            selm[t] |= (on ? 1u : 0u) << e;
        }
    }

    // Workgroup 0: the optional outputs q, s and the index list.
    if (tile == 0) {
#pragma unroll
        for (int t = 0; t < BT; ++t) {
            if (t >= ntok) break;   // uniform
            if (a.xq != nullptr) {
#pragma unroll
                for (int q = 0; q < E / 4; ++q) {
                    if (4 * q >= nvalid) break;
                    uint32_t pk = 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) pk |= ((uint32_t)qv[t][4 * q + i] & 0xFFu) << (8 * i);
                    *reinterpret_cast<uint32_t*>(a.xq + (int64_t)t * d + tid * E + 4 * q) = pk;
                }
            }
            if (a.xscale != nullptr && tid == 0) a.xscale[t] = scale[t];
            if (a.idx != nullptr) {
                uint32_t tot;
                uint32_t pos = rowsel::block_excl_scan<NT>((uint32_t)__popc(selm[t]), s_wsum, tid, tot);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (selm[t] & (1u << e)) a.idx[(int64_t)t * a.k + pos++] = tid * E + e;
            }
        }
    }

    // Phase 3: this thread's selected rows (CT / 4 = 4 packed bytes each).
    const uint32_t rowbytes = (uint32_t)(n_out / 4);
    const uint32_t colb = (uint32_t)(tile * (CT / 4));
    const __amdgpu_buffer_rsrc_t wr = weight_rsrc(a.wt, d * (int64_t)rowbytes);
    uint32_t um = 0;
#pragma unroll
    for (int t = 0; t < BT; ++t) um |= selm[t];
    uint32_t wseg[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        wseg[e] = __builtin_amdgcn_raw_buffer_load_b32(
            wr, (um >> e) & 1u ? (uint32_t)(tid * E + e) * rowbytes + colb : kOOB, 0, 0);
    int32_t acc[BT][CT];
#pragma unroll
    for (int t = 0; t < BT; ++t)
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[t][c] = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        int32_t qq[BT];
#pragma unroll
        for (int t = 0; t < BT; ++t) qq[t] = (selm[t] >> e) & 1u ? qv[t][e] : 0;
#pragma unroll
        for (int f = 0; f < 16; ++f) {
            const int32_t tv = __builtin_amdgcn_sbfe(wseg[e], 2 * f, 2);   // 00 0, 01 +1, 11 -1
#pragma unroll
            for (int t = 0; t < BT; ++t) acc[t][f] += qq[t] * tv;
        }
    }

    // Phase 4: exact sums over the threads.  Inside each wavefront a
    // butterfly over the lane bits, high bit first: while a lane holds more
    // than one value it keeps half of them (the upper half where the lane
    // bit is set) and adds its partner's copy of that half, so after
    // log2(NV) steps lane l holds value l >> (6 - log2 NV), summed over the
    // lanes that differ in those bits; the remaining steps add the rest.  The
    // wavefronts' totals are then added in LDS (integer sums: the same in any
    // order).
    constexpr int NV = BT * CT;
    static_assert(NV == 16 || NV == 32 || NV == 64, "one value per lane group");
    int32_t cur[NV];
#pragma unroll
    for (int t = 0; t < BT; ++t)
#pragma unroll
        for (int c = 0; c < CT; ++c) cur[t * CT + c] = acc[t][c];
    i8_butterfly<NV, 5>(cur, lane);
    constexpr int LG = NV == 16 ? 4 : NV == 32 ? 5 : 6;
    if ((lane & ((1 << (6 - LG)) - 1)) == 0) s_part[wave][lane >> (6 - LG)] = cur[0];
    __syncthreads();
    if (tid < NV) {
        int32_t sum = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += s_part[w][tid];
        const int t = tid / CT, c = tid % CT;
        const int64_t col = (int64_t)tile * CT + c;
        if (t < ntok && col < n_out) {
            if (a.acc != nullptr) a.acc[(int64_t)t * n_out + col] = sum;
            if (a.y != nullptr)
                a.y[(int64_t)t * n_out + col] = __fmul_rn((float)sum, __fdiv_rn(a.alpha, scale[t]));
        }
    }
}

template <int BT>
__global__ __launch_bounds__(kNT) void i8t_gemv_kernel(I8tArgs a, int cand, int nsplit) {
    constexpr int BATCH = kI8NSlot * kUnroll;
    constexpr int NCH = kI8MaxCand / kNT;   // candidate chunks per thread
    constexpr int OPT = BT * kI8CT / kNT;   // outputs per thread in the split sum
    extern __shared__ int ismem[];
    int* s_coef = ismem;                                                   // [cand+3 BATCH][BT]
    uint32_t* s_off = reinterpret_cast<uint32_t*>(ismem + (size_t)(cand + 3 * BATCH) * BT);
    __shared__ int s_wcnt[4];
    __shared__ int s_last;

    const int tile = blockIdx.x, split = blockIdx.y, tt = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t rows = a.rows, d_in = a.d_in, n_out = a.n_out;
    const int64_t j0 = (int64_t)split * cand;
    const int64_t j1 = min(d_in, j0 + (int64_t)cand);
    const int64_t tok0 = (int64_t)tt * BT;

    // Rows of [j0, j1) with a nonzero q for some token of the tile: all loads
    // issued at once, placed by one block scan in (thread, chunk) order.
    const uint32_t rowbytes = (uint32_t)(n_out / 4);
    const int64_t ntok = min((int64_t)BT, rows - tok0);
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(a.qs + tok0 * d_in), (short)0, (int)(ntok * d_in), 0x00020000);
    int c[NCH][BT];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const int64_t j = j0 + ch * kNT + tid;
        const bool jin = j < j1;
#pragma unroll
        for (int t = 0; t < BT; ++t)
            c[ch][t] = (int)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(
                qr, jin ? (uint32_t)(t * d_in + j) : kOOB, 0, 0);
    }
    uint32_t selbits = 0;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        bool any = false;
#pragma unroll
        for (int t = 0; t < BT; ++t) any = any || (c[ch][t] != 0);
        selbits |= (any ? 1u : 0u) << ch;
    }
    const uint32_t mycnt = (uint32_t)__popc(selbits);
    const uint32_t incl = wave_incl_scan_u32(mycnt);
    if (lane == 63) s_wcnt[wave] = (int)incl;
    __syncthreads();
    int before = 0, nact = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int cw = s_wcnt[w];
        if (w < wave) before += cw;
        nact += cw;
    }
    int pos = before + (int)(incl - mycnt);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        if (selbits & (1u << ch)) {
            s_off[pos] = (uint32_t)(j0 + ch * kNT + tid) * rowbytes;
#pragma unroll
            for (int t = 0; t < BT; ++t) s_coef[pos * BT + t] = c[ch][t];
            ++pos;
        }
    }
    const int nbatch = (nact + BATCH - 1) / BATCH;
    const int npad = ((nbatch + 1) / 2 * 2 + 1) * BATCH;
    for (int i = nact + tid; i < npad; i += kNT) {
        s_off[i] = kOOB;
#pragma unroll
        for (int t = 0; t < BT; ++t) s_coef[i * BT + t] = 0;
    }
    __syncthreads();

    const int slot = wave * (64 / kI8LPR) + lane / kI8LPR;
    const int64_t col = (int64_t)tile * kI8CT + (lane % kI8LPR) * kI8EPT;
    // Rows are only 4-byte aligned when n_out % 32 != 0: two dword loads; the
    // second is out of range (zero) for the last 16 columns of such a row.
    const uint32_t colb = col < n_out ? (uint32_t)(col / 4) : kOOB;
    const uint32_t colb2 = col + 16 < n_out ? (uint32_t)(col / 4 + 4) : kOOB;
    const __amdgpu_buffer_rsrc_t rs = weight_rsrc(a.wt, a.d_in * (int64_t)rowbytes);

    int acc[BT][kI8EPT];
#pragma unroll
    for (int t = 0; t < BT; ++t)
#pragma unroll
        for (int e = 0; e < kI8EPT; ++e) acc[t][e] = 0;

    u32x2 bufa[kUnroll], bufb[kUnroll];
    auto load_stage = [&](u32x2* dst, int bi) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t ro = s_off[bi * BATCH + slot + u * kI8NSlot];
            dst[u].x = __builtin_amdgcn_raw_buffer_load_b32(rs, ro + colb, 0, 0);
            dst[u].y = __builtin_amdgcn_raw_buffer_load_b32(rs, ro + colb2, 0, 0);
        }
    };
    auto mac_stage = [&](const u32x2* src, int bi) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int ai = bi * BATCH + slot + u * kI8NSlot;
            int cf[BT];
#pragma unroll
            for (int t = 0; t < BT; ++t) cf[t] = s_coef[ai * BT + t];
#pragma unroll
            for (int e = 0; e < kI8EPT; ++e) {
                const uint32_t word = e < 16 ? src[u].x : src[u].y;
                // 2-bit two's complement field: 00 -> 0, 01 -> +1, 11 -> -1
                const int tv = __builtin_amdgcn_sbfe((int)word, (2 * e) & 31, 2);
#pragma unroll
                for (int t = 0; t < BT; ++t) acc[t][e] += cf[t] * tv;
            }
        }
    };
    // Straight-line body: stages past the list hold out-of-range offsets and
    // zero coefficients, so their loads return zero without memory traffic.
    // sched_barrier keeps each stage's loads issued before the previous
    // stage's arithmetic (the scheduler would otherwise sink them).
    load_stage(bufa, 0);
    for (int bi = 0; bi < nbatch; bi += 2) {
        load_stage(bufb, bi + 1);
        __builtin_amdgcn_sched_barrier(0);
        mac_stage(bufa, bi);
        __builtin_amdgcn_sched_barrier(0);
        load_stage(bufa, bi + 2);
        __builtin_amdgcn_sched_barrier(0);
        mac_stage(bufb, bi + 1);
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();

    // Integer partial sums are exact, so only the epilogue needs an order.
    int* s_red = ismem;   // [kI8NSlot][CT] per token
    const int cl = (lane % kI8LPR) * kI8EPT;
    auto finish = [&](int64_t row, int64_t cg, int sum) {
        if (a.acc) a.acc[row * n_out + cg] = sum;
        if (a.y) a.y[row * n_out + cg] = __fmul_rn((float)sum, __fdiv_rn(a.alpha, a.xscale[row]));
    };
#pragma unroll
    for (int t = 0; t < BT; ++t) {
#pragma unroll
        for (int e = 0; e < kI8EPT; ++e) s_red[slot * kI8CT + cl + e] = acc[t][e];
        __syncthreads();
        {
            const int o = tid;   // kI8CT == kNT: one column per thread
            int sum = 0;
#pragma unroll
            for (int sl = 0; sl < kI8NSlot; ++sl) sum += s_red[sl * kI8CT + o];
            const int64_t row = tok0 + t;
            const int64_t cg = (int64_t)tile * kI8CT + o;
            if (row < rows && cg < n_out) {
                if (nsplit == 1) finish(row, cg, sum);
                else store_agent(&a.partial[((int64_t)split * rows + row) * n_out + cg], sum);
            }
        }
        __syncthreads();
    }

    // The last split of the tile sums the partials; the loads of all of a
    // thread's outputs for 8 splits are in flight together.
    if (nsplit > 1) {
        const int ci = tt * gridDim.x + tile;
        if (last_split_arrived(&a.counters[ci], nsplit, &s_last)) {
            const int64_t stride = rows * n_out;
            int64_t base[OPT];
            bool ok[OPT];
            int sum[OPT];
#pragma unroll
            for (int q = 0; q < OPT; ++q) {
                const int o = q * kNT + tid;
                const int64_t row = tok0 + o / kI8CT, cg = (int64_t)tile * kI8CT + (o % kI8CT);
                ok[q] = row < rows && cg < n_out;
                base[q] = ok[q] ? row * n_out + cg : 0;
                sum[q] = 0;
            }
            for (int sp0 = 0; sp0 < nsplit; sp0 += 8) {
                int v[8][OPT];
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int q = 0; q < OPT; ++q)
                        v[u][q] = (sp0 + u < nsplit && ok[q])
                                      ? load_agent(a.partial + (int64_t)(sp0 + u) * stride + base[q]) : 0;
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int q = 0; q < OPT; ++q) sum[q] += v[u][q];
            }
#pragma unroll
            for (int q = 0; q < OPT; ++q) {
                const int o = q * kNT + tid;
                if (ok[q]) finish(tok0 + o / kI8CT, (int64_t)tile * kI8CT + (o % kI8CT), sum[q]);
            }
            if (tid == 0) store_agent(&a.counters[ci], 0);
        }
    }
}

// ---------------------------------------------------------------------------
// Ternary x int8 on the int8 matrix cores, for token batches (16 and more):
// the union of the batch's selections covers nearly every input feature, so
// acc = Qs . T^T is a dense int8 contraction (Qs = the masked q, zeros where
// not selected).  v_mfma_i32_32x32x32_i8 sums exactly in int32, so the
// result is the same integer as any other order.
// Workgroup: 64 tokens (two 32-row MFMA tiles) x 128 outputs (one 32-column
// tile per wavefront) over a split of kT8Steps steps of 128 input features.
// Every global load of the split is issued at the start (per thread and
// step: 32 bytes of Qs and 16 packed bytes), so the steps only wait for data
// already in flight.  Per step the workgroup stages A (64 tokens x 128
// features, int8) and the decoded B tile ([k][n] int8, 128 x 128) in LDS; B
// rows have a 144-byte pitch so that the eight rows a transposing read
// touches land on distinct banks, and each wavefront takes its B operand with
// ds_read_b64_tr_b8 (in each group of 16 lanes, lane 2e + h addresses k-row
// e, columns 8h .. 8h + 7; lane j receives column j's eight k values).
// ---------------------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
constexpr int kT8CT = 128;     // output columns per workgroup
constexpr int kT8MT = 64;      // tokens per workgroup
constexpr int kT8KS = 128;     // features per step
constexpr int kT8Steps = 8;    // steps per split
constexpr int kT8Pitch = 144;  // LDS bytes per decoded k-row
constexpr int kT8APitch = 144; // LDS bytes per staged token row (128 + 16: conflict-free 16-byte reads)
constexpr int kSc1 = 16;       // buffer cache policy sc1 (agent-scope coherent)

__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* base, int byte_off) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(base + byte_off));
#else
    (void)base; (void)byte_off;
    return i32x2{0, 0};
#endif
}

// One packed byte (4 ternary weights, 2-bit two's complement: 00 = 0,
// 01 = +1, 11 = -1) -> 4 int8 in one word.  The even and the odd fields are
// spread into their bytes by one multiply each (the shifted copies do not
// overlap, so no carries), then bit 1 of each byte, set only for -1, fills
// the byte's upper bits.
__device__ __forceinline__ uint32_t decode_ternary4(uint32_t b) {
    uint32_t y = (((b & 0x33u) * 0x1001u) & 0x00030003u) | (((b & 0xCCu) * 0x40040u) & 0x03000300u);
    return y | ((y & 0x02020202u) * 0x7Fu);
}

__global__ __launch_bounds__(kNT) void i8t_mfma_kernel(I8tArgs a, int nsplit) {
    __shared__ __attribute__((aligned(16))) uint8_t s_b[2][kT8KS * kT8Pitch];
    __shared__ __attribute__((aligned(16))) uint8_t s_a[2][kT8MT * kT8APitch];
    __shared__ int s_last;
    __shared__ float s_fac[kT8MT];    // fl32(alpha / s_r) of the tile's tokens
    const int tile = blockIdx.x, split = blockIdx.y, mt = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t rows = a.rows, d_in = a.d_in, n_out = a.n_out;
    const int64_t m0 = (int64_t)mt * kT8MT, n0 = (int64_t)tile * kT8CT;
    const int64_t k_begin = (int64_t)split * kT8Steps * kT8KS;
    const int64_t k_end = min(d_in, k_begin + (int64_t)kT8Steps * kT8KS);
    const int64_t pbytes = n_out / 4;                       // packed bytes per row
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(a.qs), (short)0, (int)(rows * d_in), 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.wt), (short)0, (int)(d_in * pbytes), 0x00020000);

    // Thread t stages token row t / 4, features 32 (t % 4) .. +31 of a step,
    // and packed k-row t / 2, bytes 16 (t % 2) .. +15 (64 columns) of the tile.
    const int arow_l = tid >> 2, aq = tid & 3, prow = tid >> 1, pq = tid & 1;
    const int64_t arow = m0 + arow_l;
    const int64_t pbyte = n0 / 4 + 16 * pq;
    uint32_t aoff[kT8Steps], poff[kT8Steps];
#pragma unroll
    for (int s = 0; s < kT8Steps; ++s) {
        const int64_t ka = k_begin + (int64_t)s * kT8KS + 32 * aq;
        const int64_t kp = k_begin + (int64_t)s * kT8KS + prow;
        aoff[s] = (arow < rows && ka < k_end) ? (uint32_t)(arow * d_in + ka) : kOOB;
        poff[s] = (kp < k_end && pbyte < pbytes) ? (uint32_t)(kp * pbytes + pbyte) : kOOB;
    }
    u32x4 ra[kT8Steps][2], rp[kT8Steps];
#pragma unroll
    for (int s = 0; s < kT8Steps; ++s) {
        rp[s] = __builtin_amdgcn_raw_buffer_load_b128(wr, poff[s], 0, 0);
        ra[s][0] = __builtin_amdgcn_raw_buffer_load_b128(qr, aoff[s], 0, 0);
        ra[s][1] = __builtin_amdgcn_raw_buffer_load_b128(qr, aoff[s] == kOOB ? kOOB : aoff[s] + 16u, 0, 0);
    }
    auto stage = [&](int buf, int s) {
        u32x4* ad = reinterpret_cast<u32x4*>(&s_a[buf][arow_l * kT8APitch + 32 * aq]);
        ad[0] = ra[s][0];
        ad[1] = ra[s][1];
        uint8_t* dst = &s_b[buf][prow * kT8Pitch + 64 * pq];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t v = rp[s][w];
            *reinterpret_cast<uint4*>(dst + 16 * w) =
                make_uint4(decode_ternary4(v & 0xFFu), decode_ternary4((v >> 8) & 0xFFu),
                           decode_ternary4((v >> 16) & 0xFFu), decode_ternary4(v >> 24));
        }
    };
    // Fragment reads (four 32-feature slices per step).  A: lane -> token row
    // 32 i + lane % 32, features 32 sl + 16 (lane / 32) .. +15.  B: lane group
    // g = lane / 16 covers columns 32 wave + 16 (g % 2) .. +15 and features
    // 32 sl + 16 (g / 2) .. +15.
    const int g = lane >> 4, li = lane & 15;
    const int trow = 16 * (g >> 1) + (li >> 1);
    const int tcol = 32 * wave + 16 * (g & 1) + 8 * (li & 1);

    i32x16 acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0;

    stage(0, 0);
    __syncthreads();
    // All kT8Steps steps run (steps past the split's features read zeros), so
    // the loop unrolls fully and the prefetched registers stay registers.
#pragma unroll
    for (int st = 0; st < kT8Steps; ++st) {
        const int cb = st & 1;
        i32x4 afr[2][4], bfr[4];
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
            const int off = (32 * sl + trow) * kT8Pitch + tcol;
            const i32x2 lo = lds_read_tr8(s_b[cb], off), hi = lds_read_tr8(s_b[cb], off + 8 * kT8Pitch);
            bfr[sl] = i32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
            for (int i = 0; i < 2; ++i)
                afr[i][sl] = __builtin_bit_cast(i32x4, *reinterpret_cast<const u32x4*>(
                    &s_a[cb][(32 * i + (lane & 31)) * kT8APitch + 32 * sl + 16 * (lane >> 5)]));
        }
        // The next step goes into the other buffers (last read before the
        // previous barrier) while the MFMAs run.
        if (st + 1 < kT8Steps) stage(cb ^ 1, st + 1);
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(afr[i][sl], bfr[sl], acc[i], 0, 0, 0);
        __syncthreads();
    }

    // Outputs: acc[i][v] is token m0 + 32 i + 8 (v / 4) + 4 (lane / 32) + v % 4,
    // column n0 + 32 wave + lane % 32.
    const int64_t col = n0 + 32 * wave + (lane & 31);
    // Dequantisation factors, one per token row of the tile (staged before
    // any output is written, so no output waits on its own scale load).
    auto stage_factors = [&]() {
        if (a.y != nullptr && tid < kT8MT) {
            const int64_t r = m0 + tid;
            s_fac[tid] = r < rows ? __fdiv_rn(a.alpha, a.xscale[r]) : 0.0f;
        }
        __syncthreads();
    };
    auto finish = [&](int64_t row, int sum) {
        if (a.acc) a.acc[row * n_out + col] = sum;
        if (a.y) a.y[row * n_out + col] = __fmul_rn((float)sum, s_fac[row - m0]);
    };
    auto out_row = [&](int i, int v) -> int64_t {
        return m0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    };
    if (nsplit == 1) {
        stage_factors();
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = out_row(i, v);
                if (row < rows && col < n_out) finish(row, acc[i][v]);
            }
        return;
    }
    // Splits: add into the zeroed int32 sums (integer addition, so the result
    // does not depend on the order the splits arrive in); the last split of
    // the tile then dequantises (with factors staged before the handoff).
    stage_factors();
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t row = out_row(i, v);
            if (row < rows && col < n_out)
                __hip_atomic_fetch_add(&a.acc_sum[row * n_out + col], (int32_t)acc[i][v], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
    const int ci = mt * gridDim.x + tile;
    if (last_split_arrived(&a.counters[ci], nsplit, &s_last)) {
        if (a.y != nullptr) {
            // Buffer loads with 32-bit offsets (entries past the batch or the
            // outputs take the out-of-range offset and read 0), unconditional
            // so that all of a thread's loads are in flight together; cache
            // policy sc1: agent-coherent, as other workgroups added the sums.
            const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
                a.acc_sum, (short)0, (int)(rows * n_out * 4), 0x00020000);
            int sum[2][16];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t row = out_row(i, v);
                    const bool ok = row < rows && col < n_out;
                    sum[i][v] = (int)__builtin_amdgcn_raw_buffer_load_b32(
                        sr, ok ? (uint32_t)((row * n_out + col) * 4) : kOOB, 0, kSc1);
                }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t row = out_row(i, v);
                    if (row < rows && col < n_out)
                        a.y[row * n_out + col] = __fmul_rn((float)sum[i][v], s_fac[row - m0]);
                }
        }
        if (tid == 0) store_agent(&a.counters[ci], 0);
    }
}

}  // namespace

GemvPlan plan_gemv(int64_t rows, int64_t d_in, int64_t n_out, int w_is_bf16, int max_bt,
                   int64_t target) {
    GemvPlan p{};
    p.lpr = kLPR;
    p.ept = w_is_bf16 ? 8 : 4;
    p.bt = pow2_tile(rows, max_bt);
    // 16-token tiles run an MFMA kernel: bf16 weights in 64-column tiles on the
    // bf16 matrix cores, fp32 weights in 16 * EPT-column tiles on the fp32 ones.
    // With bf16 weights, 8 tokens also take the bf16 MFMA kernel (as a half-empty
    // 16-token tile): it beats eight fp32 FMAs per weight.
    if (w_is_bf16 && p.bt == 8) p.bt = 16;
    const bool bmfma = p.bt == 16 && w_is_bf16;
    p.ct = bmfma ? kBCols : p.bt == 16 ? 16 * p.ept : kFLPR * p.ept;
    p.n_tiles = (int)ceil_div(n_out, p.ct);
    p.n_tok_tiles = (int)ceil_div(rows, p.bt);
    const int64_t base = (int64_t)p.n_tiles * p.n_tok_tiles;
    int64_t cand;
    if (bmfma) {
        // As many splits as keep every workgroup resident at once (three per
        // CU), in whole 4-group stages.
        const int64_t cap = 768;
        int64_t ns = cap / base;
        if (ns < 1) ns = 1;
        cand = ceil_div(ceil_div(d_in, ns), 4 * kBGroup) * 4 * kBGroup;
    } else {
        // The FMA kernels stage <= 32 KB of coefficients in LDS.
        const int cand_max = 8192 / p.bt < kFMaxCand ? 8192 / p.bt : kFMaxCand;
        int64_t ns = ceil_div(target > 0 ? target : kGemvTargetWG, base);
        if (ns < 1) ns = 1;
        cand = ceil_div(ceil_div(d_in, ns), 64) * 64;
        if (cand > cand_max) cand = cand_max;
        if (cand < 64) cand = 64;
    }
    p.cand = (int)cand;
    p.nsplit = (int)ceil_div(d_in, cand);
    if (p.nsplit < 1) p.nsplit = 1;
    p.partial_floats = p.nsplit > 1 ? (size_t)p.nsplit * rows * n_out : 0;
    p.prep_bytes = bmfma ? bfrag_bytes(d_in, p.n_tok_tiles) : 0;
    p.scratch_floats = (p.partial_floats * 4 + 255) / 256 * 64 + (p.prep_bytes + 3) / 4;
    p.n_counters = p.n_tiles * p.n_tok_tiles;
    return p;
}

// Forming the fragments inside the gather converts each group once per column
// tile instead of once, but saves the packing launch: it pays for a half-empty
// tile (8 tokens: 65.4 us per Llama-7B FFN step against 67.1), not for a full
// one (69.2 against 68.6).
bool bmfma_fused(int64_t rows) { return rows <= 8; }

// Records written by the selection launch beat both the packing launch and
// the fused conversion from 8 tokens on (Llama-7B FFN step at 8 tokens: 61.0
// us against 61.7 fused; at 6 tokens 60.3 against 59.9).
bool gemv_takes_records(const GemvPlan& p, int w_is_bf16, int64_t rows) {
    return p.bt == 16 && w_is_bf16 && (rows >= 8 || !bmfma_fused(rows));
}

void* gemv_records(const GemvPlan& p, float* partial, int64_t d_in, int64_t* groups) {
    const BFrag bf = bfrag_carve(reinterpret_cast<char*>(partial) + (p.partial_floats * 4 + 255) / 256 * 256,
                                 d_in, p.n_tok_tiles);
    *groups = bf.groups;
    return bf.frag;
}

bool gemv_accumulate_supported(const GemvPlan& p, int w_is_bf16) {
    return !(p.bt == 16 && !w_is_bf16);
}

// A row pitch is 0 (n_out) or at least n_out, in whole 16-byte units.
static bool gemv_pitch_ok(const GemvArgs& a, int w_is_bf16) {
    return a.w_ld == 0 || (a.w_ld >= a.n_out && a.w_ld % (w_is_bf16 ? 8 : 4) == 0);
}

hipError_t launch_gemv(const GemvPlan& p, int w_is_bf16, const GemvArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    if (!gemv_pitch_ok(a, w_is_bf16)) return hipErrorInvalidValue;
    // The descriptor form exists in the FMA kernel (tiles of at most eight tokens).
    if (a.sel_desc != nullptr && p.bt > 8) return hipErrorInvalidValue;
    if (a.accumulate && (a.y_bf16 || a.epilogue != EPI_STORE || !gemv_accumulate_supported(p, w_is_bf16)))
        return hipErrorInvalidValue;
    if (a.row_out != nullptr && (!a.accumulate || p.bt != 1 || a.row_scale == nullptr))
        return hipErrorInvalidValue;
    const int ept = w_is_bf16 ? 8 : 4;
    const int ct = kFLPR * ept;
    const int tg = p.bt < 2 ? p.bt : 2;
    dim3 grid(p.n_tiles, p.nsplit, p.n_tok_tiles);
    if (p.bt == 16 && w_is_bf16) {
        const BFrag bf = bfrag_carve(reinterpret_cast<char*>(a.partial) + (p.partial_floats * 4 + 255) / 256 * 256,
                                     a.d_in, p.n_tok_tiles);
        const int use_lo = a.xs_bf16 ? 0 : 1;
        if (a.frag_ready == 2) {   // records from the selection launch
            gather_bmfma_kernel<2><<<grid, dim3(kNT), 0, stream>>>(a, bf, p.cand, p.nsplit, use_lo);
            return hipGetLastError();
        }
        if (bmfma_fused(a.rows)) {
            gather_bmfma_kernel<1><<<grid, dim3(kNT), 0, stream>>>(a, bf, p.cand, p.nsplit, use_lo);
            return hipGetLastError();
        }
        if (!a.frag_ready)
            bfrag_kernel<<<dim3((unsigned)ceil_div(bf.groups, 4), p.n_tok_tiles), dim3(kNT), 0, stream>>>(
                a.xs, a.rows, a.d_in, use_lo, bf);
        gather_bmfma_kernel<0><<<grid, dim3(kNT), 0, stream>>>(a, bf, p.cand, p.nsplit, use_lo);
        return hipGetLastError();
    }
    if (p.bt == 16) {
        const size_t padded = (size_t)p.cand + 3 * 64;
        size_t lds = padded * 16 * 4 + padded * 4;
        const size_t lds_red = (size_t)4 * 16 * 16 * ept * 4;
        if (lds_red > lds) lds = lds_red;
        if (w_is_bf16) gather_mfma_kernel<1><<<grid, dim3(kNT), lds, stream>>>(a, p.cand, p.nsplit);
        else gather_mfma_kernel<0><<<grid, dim3(kNT), lds, stream>>>(a, p.cand, p.nsplit);
        return hipGetLastError();
    }
    const size_t padded = (size_t)p.cand + 3 * kFNSlot * kMaxUnroll;
    size_t lds_a = padded * p.bt * 4 + padded * 4;
    size_t lds_c = (size_t)kFNSlot * tg * ct * 4;
    size_t lds = lds_a > lds_c ? lds_a : lds_c;
#define QS_GEMV_CASE(WB, BTV)                                                              \
    if (w_is_bf16 == WB && p.bt == BTV) {                                                  \
        gather_gemv_kernel<WB, BTV><<<grid, dim3(kNT), lds, stream>>>(a, p.cand, p.nsplit); \
        return hipGetLastError();                                                          \
    }
    QS_GEMV_CASE(1, 1) QS_GEMV_CASE(1, 2) QS_GEMV_CASE(1, 4) QS_GEMV_CASE(1, 8)
    QS_GEMV_CASE(0, 1) QS_GEMV_CASE(0, 2) QS_GEMV_CASE(0, 4) QS_GEMV_CASE(0, 8)
#undef QS_GEMV_CASE
    return hipErrorInvalidValue;
}

bool gather_sel_supported(int64_t rows, int64_t d_in, int64_t n_out) {
    return rows >= 1 && rows <= 65535 && desc31_supported(d_in) && n_out % 8 == 0 && n_out > 0;
}

void gather_sel_plan(int64_t d_in, int64_t n_out, int* n_tiles, int* nsplit, int* cand) {
    const int64_t nt = ceil_div(n_out, kFsCols);
    int64_t ns = ceil_div(256, nt);   // one workgroup per CU
    const int64_t ns_min = ceil_div(d_in, kFsMaxCand);
    if (ns < ns_min) ns = ns_min;
    int64_t cd = ceil_div(ceil_div(d_in, ns), 64) * 64;
    if (cd > kFsMaxCand) cd = kFsMaxCand;
    *n_tiles = (int)nt;
    *cand = (int)cd;
    *nsplit = (int)ceil_div(d_in, cd);
}

hipError_t launch_gather_sel(const GemvArgs& a, hipStream_t stream) {
    if (!gather_sel_supported(a.rows, a.d_in, a.n_out) || a.sel_desc != nullptr ||
        a.epilogue != EPI_STORE || (a.accumulate && a.y_bf16) || (!a.accumulate && a.rows != 1) ||
        (a.w_ld != 0 && (a.w_ld < a.n_out || a.w_ld % 8 != 0)))
        return hipErrorInvalidValue;
    int nt, ns, cand;
    gather_sel_plan(a.d_in, a.n_out, &nt, &ns, &cand);
    const int nq = (int)ceil_div(a.d_in, 4 * kFsNT);
    const dim3 grid((unsigned)nt, (unsigned)ns, (unsigned)a.rows), block(kFsNT);
#define QS_FS_CASE(NQV)                                                                   \
    if (nq <= NQV) {                                                                      \
        gather_sel_kernel<NQV><<<grid, block, (size_t)fs_lds_words<NQV>() * 4, stream>>>(a, cand, ns); \
        return hipGetLastError();                                                         \
    }
    QS_FS_CASE(1) QS_FS_CASE(2) QS_FS_CASE(3) QS_FS_CASE(4)
#undef QS_FS_CASE
    return hipErrorInvalidValue;
}

bool up_cols_supported(int64_t rows, int64_t d, int64_t ffn) {
    if (!(rows >= 1 && rows <= 4 && d % 8 == 0 && d <= kUpColsMaxD && ffn % 8 == 0 &&
          ffn <= kUpColsMaxFfn))
        return false;
    // The row lists must fit in the 160 KiB of LDS (for a tile of four
    // tokens: d <= 4096).
    const bool e8 = d <= 8 * kUcNT;
    int64_t words = 0;
    if (rows == 1) {
        const int64_t w1 = e8 ? uc_lds_words<1, 8, false>() : uc_lds_words<1, 16, false>();
        const int64_t w2 = uc_lds_tail<1, true>(d) + 16;
        words = w1 > w2 ? w1 : w2;
    } else {
        words = rows == 2 ? uc_lds_tail<2, true>(d) + 16 : uc_lds_tail<4, true>(d) + 16;
    }
    return words * 4 <= 160 * 1024;
}

hipError_t launch_up_cols(const UpColsArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    if (!up_cols_supported(a.rows, a.d, a.ffn) || (a.h == nullptr) == (a.hb == nullptr) ||
        (a.linear && a.w2 != nullptr) || (a.w_ld != 0 && (a.w_ld < a.ffn || a.w_ld % 8 != 0)))
        return hipErrorInvalidValue;
    const int bt = a.rows == 1 ? 1 : a.rows == 2 ? 2 : 4;
    if (a.zero != nullptr && a.n_zero % 4 != 0) return hipErrorInvalidValue;
    const int e = a.d <= 8 * kUcNT ? 8 : 16;
    // One 64-column tile (128 bytes of each row) per workgroup.  (Spreading
    // the columns evenly over 256 workgroups, 40 or 48 each, was slower: the
    // row segments then straddle 128-byte lines that two workgroups fetch.)
    const dim3 grid((unsigned)ceil_div(a.ffn, kUcCols), (unsigned)ceil_div(a.rows, bt));
    const bool dual = a.w2 != nullptr;
#define QS_UC_CASE(BTV, EV, DU)                                                          \
    if (bt == BTV && e == EV && dual == DU) {                                            \
        const size_t lds = (size_t)(BTV == 1 && !DU ? uc_lds_words<BTV, EV, DU>()       \
                                                    : uc_lds_tail<BTV, DU>(a.d) + 16) * 4; \
        up_cols_kernel<BTV, EV, DU><<<grid, dim3(kUcNT), lds, stream>>>(a);              \
        return hipGetLastError();                                                        \
    }
#define QS_UC_E(BTV, DU) QS_UC_CASE(BTV, 8, DU) QS_UC_CASE(BTV, 16, DU)
    QS_UC_E(1, false) QS_UC_E(2, false) QS_UC_E(4, false)
    QS_UC_E(1, true) QS_UC_E(2, true) QS_UC_E(4, true)
#undef QS_UC_E
#undef QS_UC_CASE
    return hipErrorInvalidValue;
}

bool gemv_dual_supported(const GemvPlan& p, int w_is_bf16) {
    return p.bt == 1 || p.bt == 2 || p.bt == 4 || (p.bt == 16 && w_is_bf16);
}

hipError_t launch_gemv_dual(const GemvPlan& p, int w_is_bf16, const GemvArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    if (!gemv_pitch_ok(a, w_is_bf16)) return hipErrorInvalidValue;
    if (!gemv_dual_supported(p, w_is_bf16) || a.w2 == nullptr || a.row_expert != nullptr ||
        (a.accumulate ? a.y2 == nullptr : p.nsplit > 1 && a.partial2 == nullptr))
        return hipErrorNotSupported;
    if (p.bt == 16) {   // bf16 weights: the 16-token MFMA gather with both matrices
        const dim3 grid(p.n_tiles, p.nsplit, p.n_tok_tiles);
        const BFrag bf = bfrag_carve(reinterpret_cast<char*>(a.partial) + (p.partial_floats * 4 + 255) / 256 * 256,
                                     a.d_in, p.n_tok_tiles);
        const int use_lo = a.xs_bf16 ? 0 : 1;
        if (a.frag_ready == 2) return hipErrorNotSupported;   // records come with masks here
        if (bmfma_fused(a.rows)) {
            gather_bmfma_kernel<1, true><<<grid, dim3(kNT), 0, stream>>>(a, bf, p.cand, p.nsplit, use_lo);
            return hipGetLastError();
        }
        bfrag_kernel<<<dim3((unsigned)ceil_div(bf.groups, 4), p.n_tok_tiles), dim3(kNT), 0, stream>>>(
            a.xs, a.rows, a.d_in, use_lo, bf);
        gather_bmfma_kernel<0, true><<<grid, dim3(kNT), 0, stream>>>(a, bf, p.cand, p.nsplit, use_lo);
        return hipGetLastError();
    }
    const int ept = w_is_bf16 ? 8 : 4;
    const int ct = kFLPR * ept;
    const int tg = p.bt < 2 ? p.bt : 2;
    const dim3 grid(p.n_tiles, p.nsplit, p.n_tok_tiles);
    const size_t padded = (size_t)p.cand + 3 * kFNSlot * kUnroll;
    const size_t lds_a = padded * p.bt * 4 + padded * 4;
    const size_t lds_c = (size_t)kFNSlot * tg * ct * 4;
    const size_t lds = lds_a > lds_c ? lds_a : lds_c;
#define QS_GEMV_DUAL_CASE(WB, BTV)                                                                \
    if (w_is_bf16 == WB && p.bt == BTV) {                                                         \
        gather_gemv_kernel<WB, BTV, true><<<grid, dim3(kNT), lds, stream>>>(a, p.cand, p.nsplit); \
        return hipGetLastError();                                                                 \
    }
    QS_GEMV_DUAL_CASE(1, 1) QS_GEMV_DUAL_CASE(1, 2) QS_GEMV_DUAL_CASE(1, 4)
    QS_GEMV_DUAL_CASE(0, 1) QS_GEMV_DUAL_CASE(0, 2) QS_GEMV_DUAL_CASE(0, 4)
#undef QS_GEMV_DUAL_CASE
    return hipErrorNotSupported;
}

I8tPlan plan_i8t(int64_t rows, int64_t d_in, int64_t n_out) {
    I8tPlan p{};
    // (The int32 sums are addressed with 32-bit buffer offsets below the
    // out-of-range offset: at most 2^30 bytes.)
    if (rows >= 16 && d_in % 16 == 0 && rows * n_out * 4 < (int64_t)kOOB) {
        // Token batches: the int8 matrix-core kernel, 64 x 128 tiles, the
        // features split into runs of 1024.
        p.mfma = 1;
        p.ct = kT8CT;
        p.n_tiles = (int)ceil_div(n_out, kT8CT);
        p.bt = kT8MT;
        p.n_tok_tiles = (int)ceil_div(rows, kT8MT);
        p.cand = kT8Steps * kT8KS;
        p.nsplit = (int)ceil_div(d_in, p.cand);
        p.partial_ints = p.nsplit > 1 ? (size_t)rows * n_out : 0;   // the int32 sums
        p.n_counters = p.n_tiles * p.n_tok_tiles;
        return p;
    }
    p.ct = kI8CT;
    p.n_tiles = (int)ceil_div(n_out, p.ct);
    p.bt = pow2_tile(rows, 2);   // 32 int32 accumulators per token per lane
    p.n_tok_tiles = (int)ceil_div(rows, p.bt);
    const int cand_max = kI8MaxCand;
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

bool i8t_fused_supported(int64_t rows, int64_t d_in, int64_t n_out) {
    return rows >= 1 && rows <= 4 && d_in % 4 == 0 && d_in <= 16 * i8f_threads(rows == 1 ? 1 : 2) &&
           n_out % 16 == 0;
}

hipError_t launch_i8t_fused(const I8fArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    if (!i8t_fused_supported(a.rows, a.d_in, a.n_out) || a.k < 0 || a.k > a.d_in)
        return hipErrorInvalidValue;
    const int bt = a.rows == 1 ? 1 : a.rows == 2 ? 2 : 4;
    const int nt = i8f_threads(bt);
    const int e = a.d_in <= 4 * nt ? 4 : a.d_in <= 8 * nt ? 8 : 16;
    const dim3 grid((unsigned)ceil_div(a.n_out, kI8Ct));
#define QS_I8F_CASE(BTV, EV)                                                       \
    if (bt == BTV && e == EV) {                                                    \
        i8t_fused_kernel<BTV, EV><<<grid, dim3(i8f_threads(BTV)), 0, stream>>>(a); \
        return hipGetLastError();                                                  \
    }
    QS_I8F_CASE(1, 4) QS_I8F_CASE(1, 8) QS_I8F_CASE(1, 16)
    QS_I8F_CASE(2, 4) QS_I8F_CASE(2, 8) QS_I8F_CASE(2, 16)
    QS_I8F_CASE(4, 4) QS_I8F_CASE(4, 8) QS_I8F_CASE(4, 16)
#undef QS_I8F_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_i8t(const I8tPlan& p, const I8tArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    if (p.mfma) {
        if (p.nsplit > 1 && a.acc_sum == nullptr) return hipErrorInvalidValue;
        i8t_mfma_kernel<<<dim3(p.n_tiles, p.nsplit, p.n_tok_tiles), dim3(kNT), 0, stream>>>(a, p.nsplit);
        return hipGetLastError();
    }
    const size_t padded = (size_t)p.cand + 3 * kI8NSlot * kUnroll;
    size_t lds_a = padded * p.bt * 4 + padded * 4;
    size_t lds_c = (size_t)kI8NSlot * kI8CT * 4;
    size_t lds = lds_a > lds_c ? lds_a : lds_c;
    dim3 grid(p.n_tiles, p.nsplit, p.n_tok_tiles);
#define QS_I8T_CASE(BTV)                                                                \
    if (p.bt == BTV) {                                                                  \
        i8t_gemv_kernel<BTV><<<grid, dim3(kNT), lds, stream>>>(a, p.cand, p.nsplit);    \
        return hipGetLastError();                                                       \
    }
    QS_I8T_CASE(1) QS_I8T_CASE(2)
#undef QS_I8T_CASE
    return hipErrorInvalidValue;
}

}  // namespace qs
