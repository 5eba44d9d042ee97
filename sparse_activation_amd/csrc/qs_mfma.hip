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
// The same product, pipelined, for either operand layout.  An operand is
// k-contiguous (row m holds A(m, 0..K-1), the nn.Linear layout) or k-major
// (row k holds A(0..M-1, k), e.g. activations [tokens, features] when the
// contraction runs over tokens, as in the weight gradient).  Tile
// 256 x BN x 64 per workgroup of NW wavefronts (NW / 2 x 2, each
// 256 / (NW / 2) x BN / 2).  Slices of 64 along k go global -> registers two
// slices ahead of the MFMAs and registers -> LDS (one of two buffers) one
// slice ahead, one barrier per slice.  The per-CU vector-memory path (64 bytes
// per clock) and the LDS stores would stall a wavefront for most of a slice if
// issued as a block, so each chunk's LDS store and the reload of its register
// are interleaved with the MFMAs (three MFMAs, one store, one load).
//
// LDS layouts.  k-contiguous: a row of a slice is 8 chunks of 16 bytes stored
// at chunk position c ^ ((row >> 1) & 7): with 64 four-byte banks and 16 lanes
// served per pass, the 16 rows of a fragment read's pass hit 16 distinct
// 16-byte bank groups.  k-major: the slice is stored as it lies in memory,
// 64 k-rows of BM (or BN) elements padded by 64 bytes, and fragments come from
// gfx950's transposing LDS read (ds_read_b64_tr_b16: in each group of 16
// lanes, lane 4e + q supplies the address of four consecutive elements of
// k-row e, and lane j receives element j % 4 of lane 4e + j / 4's run for
// e = 0..3, i.e. four consecutive k of column 4q + j % 4).  With the pad a
// pass of 32 lanes (4 k-rows x 64 bytes) covers 64 distinct banks.
// (Direct global -> LDS loads would save the register staging, but the
// compiler then waits for every load in flight before each LDS read.)
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x2 lds_read_tr16(const u32x4* base, int byte_off) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const char* p = reinterpret_cast<const char*>(base) + byte_off;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
#else
    (void)base; (void)byte_off;
    return u32x2{0u, 0u};
#endif
}

template <int BN, int NW, bool AK, bool BK>
__global__ __launch_bounds__(64 * NW) void gemm_bf16_deep_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, void* __restrict__ C,
    int M, int N, int K, int lda, int ldb, int c_bf16, int tiles_m, int tiles_n) {
    constexpr int NTH = 64 * NW, WM = NW / 2;              // wavefronts: WM x 2
    constexpr int BM = 256, TM = BM / WM / 32, TN = BN / 64;
    constexpr int QA = BM * 8 / NTH, QB = BN * 8 / NTH;    // 16-byte chunks per thread per slice
    static_assert(BN % 64 == 0 && (BM * 8) % NTH == 0 && (BN * 8) % NTH == 0, "tile shape");
    // LDS pitch (16-byte chunks) of a k-row in the k-major layout: a 64-byte pad
    // puts four consecutive k-rows 64 bytes apart modulo 256.
    constexpr int APITCH = BM / 8 + 4, BPITCH = BN / 8 + 4;
    static_assert((APITCH * 16) % 256 == 64 || (APITCH * 16) % 256 == 192, "A pitch");
    static_assert((BPITCH * 16) % 256 == 64 || (BPITCH * 16) % 256 == 192, "B pitch");
    constexpr int ASZ = AK ? 64 * APITCH : BM * 8;
    constexpr int BSZ = BK ? 64 * BPITCH : BN * 8;
    __shared__ u32x4 sA0[ASZ], sA1[ASZ];
    __shared__ u32x4 sB0[BSZ], sB1[BSZ];

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
    const int wm = wave >> 1, wn = wave & 1;

    // Chunk q of this thread (slot sl = q * NTH + tid).
    //  k-contiguous: LDS slot sl (row sl / 8) holds global chunk
    //    (sl % 8) ^ ((row >> 1) & 7) of that row; rows past M or N repeat the
    //    last row (their results are never stored).  kq = 8 * chunk.
    //  k-major: k-row sl / (BM / 8), chunk sl % (BM / 8) of 8 columns, stored
    //    unswizzled at pitch APITCH; chunks past M or N repeat the last chunk
    //    (M % 8 == 0).  kq = the k-row.
    // A chunk of slice kt is loaded iff 64 kt + kq < K (K % 8 == 0 when the
    // operand is k-contiguous); otherwise at an out-of-range offset, which
    // reads zeros and moves no memory.
    // kq and the LDS slot are recomputed from (q, tid) where used: with q a
    // compile-time constant they fold to a per-thread base plus a constant
    // (or a short multiply-shift), which costs fewer registers than arrays.
    auto kqa = [&](int q) -> int {
        const int sl = q * NTH + tid;
        if constexpr (!AK) return 8 * ((sl & 7) ^ (((sl >> 3) >> 1) & 7));
        else return sl / (BM / 8);
    };
    auto kqb = [&](int q) -> int {
        const int sl = q * NTH + tid;
        if constexpr (!BK) return 8 * ((sl & 7) ^ (((sl >> 3) >> 1) & 7));
        else return sl / (BN / 8);
    };
    auto lsa = [&](int q) -> int {
        const int sl = q * NTH + tid;
        if constexpr (!AK) return sl;
        else return (sl / (BM / 8)) * APITCH + sl % (BM / 8);
    };
    auto lsb = [&](int q) -> int {
        const int sl = q * NTH + tid;
        if constexpr (!BK) return sl;
        else return (sl / (BN / 8)) * BPITCH + sl % (BN / 8);
    };
    int offa[QA], offb[QB];
#pragma unroll
    for (int q = 0; q < QA; ++q) {
        const int sl = q * NTH + tid;
        if constexpr (!AK) {
            const int row = sl >> 3;
            offa[q] = min(m0 + row, M - 1) * lda + kqa(q);
        } else {
            offa[q] = kqa(q) * lda + min(m0 + 8 * (sl % (BM / 8)), M - 8);
        }
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
        const int sl = q * NTH + tid;
        if constexpr (!BK) {
            const int row = sl >> 3;
            offb[q] = min(n0 + row, N - 1) * ldb + kqb(q);
        } else {
            offb[q] = kqb(q) * ldb + min(n0 + 8 * (sl % (BN / 8)), N - 8);
        }
    }
    const uint32_t ksa = AK ? 64u * (uint32_t)lda : 64u;   // elements per slice step
    const uint32_t ksb = BK ? 64u * (uint32_t)ldb : 64u;
    const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(A), (short)0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(B), (short)0, 0x7FFFFFFF, 0x00020000);
    const int nk = (K + 63) / 64;
    // Every load and store of the loop is unconditional (slices past the end
    // load at the out-of-range offset), so the compiler's wait counts stay
    // exact across iterations.
    auto aoff = [&](int q, int kt) -> uint32_t {
        return 64 * kt + kqa(q) < K ? ((uint32_t)offa[q] + (uint32_t)kt * ksa) * 2u : 0x80000000u;
    };
    auto boff = [&](int q, int kt) -> uint32_t {
        return 64 * kt + kqb(q) < K ? ((uint32_t)offb[q] + (uint32_t)kt * ksb) * 2u : 0x80000000u;
    };
    auto gload = [&](u32x4* ra, u32x4* rb, int kt) {
#pragma unroll
        for (int q = 0; q < QA; ++q) ra[q] = __builtin_amdgcn_raw_buffer_load_b128(ar, aoff(q, kt), 0, 0);
#pragma unroll
        for (int q = 0; q < QB; ++q) rb[q] = __builtin_amdgcn_raw_buffer_load_b128(br, boff(q, kt), 0, 0);
    };
    auto lstore = [&](u32x4* sa, u32x4* sb, const u32x4* ra, const u32x4* rb) {
#pragma unroll
        for (int q = 0; q < QA; ++q) sa[lsa(q)] = ra[q];
#pragma unroll
        for (int q = 0; q < QB; ++q) sb[lsb(q)] = rb[q];
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int r32 = lane & 31, kg = lane >> 5;
    // Transposing-read addresses (k-major operands): lane group G = lane / 16
    // covers columns 16 (G % 2) .. +15 and k 8 (G / 2) .. +7 of a 32 x 16
    // fragment; lane j of the group addresses k-row j / 4 (+4 for the second
    // read) and columns 4 (j % 4) .. +3.
    const int trk = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int trc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto frag = [&](const u32x4* sa, const u32x4* sb, int ks, bf16x8* af, bf16x8* bfr) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm * (BM / WM) + i * 32;
            if constexpr (!AK) {
                const int r = row + r32, c = 2 * ks + kg;
                af[i] = as_bf16x8(sa[r * 8 + (c ^ ((r >> 1) & 7))]);
            } else {
                const int off = ((16 * ks + trk) * APITCH * 16) + (row + trc) * 2;
                const u32x2 lo = lds_read_tr16(sa, off), hi = lds_read_tr16(sa, off + 4 * APITCH * 16);
                af[i] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int row = wn * (BN / 2) + j * 32;
            if constexpr (!BK) {
                const int r = row + r32, c = 2 * ks + kg;
                bfr[j] = as_bf16x8(sb[r * 8 + (c ^ ((r >> 1) & 7))]);
            } else {
                const int off = ((16 * ks + trk) * BPITCH * 16) + (row + trc) * 2;
                const u32x2 lo = lds_read_tr16(sb, off), hi = lds_read_tr16(sb, off + 4 * BPITCH * 16);
                bfr[j] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
        }
    };
    // One slice: the MFMAs of slice kt (LDS buffer sa/sb), with the staging
    // work spread between them: item q stores chunk q of slice kt + 1 (held in
    // ra/rb) into the other buffer and reloads the register with chunk q of
    // slice kt + 3.  sched_group_barrier lays the k-step out as: its fragment
    // reads for the next k-step, then (3 MFMAs, 1 LDS store, 1 global load)
    // groups, so the per-CU load and store traffic runs under the MFMAs
    // instead of stalling the wavefront in a block of its own.
    constexpr int NI = QA + QB;            // staging items per slice
    constexpr int IPK = (NI + 3) / 4;      // items per k-step
    constexpr int NFR = TM * (AK ? 2 : 1) + TN * (BK ? 2 : 1);   // LDS reads per k-step
    constexpr int MPI = (TM * TN) / IPK;   // MFMAs before each staging item
    static_assert(MPI >= 1 && 4 * IPK >= NI, "staging schedule");
    auto item = [&](u32x4* wa, u32x4* wb, u32x4* ra, u32x4* rb, int q, int kt3) {
        if (q < QA) {
            wa[lsa(q)] = ra[q];
            ra[q] = __builtin_amdgcn_raw_buffer_load_b128(ar, aoff(q, kt3), 0, 0);
        } else {
            const int qb = q - QA;
            wb[lsb(qb)] = rb[qb];
            rb[qb] = __builtin_amdgcn_raw_buffer_load_b128(br, boff(qb, kt3), 0, 0);
        }
    };
    auto slice = [&](const u32x4* sa, const u32x4* sb, u32x4* wa, u32x4* wb, u32x4* ra, u32x4* rb, int kt3) {
        bf16x8 af[2][TM], bfr[2][TN];
        frag(sa, sb, 0, af[0], bfr[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks < 3) frag(sa, sb, ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
#pragma unroll
            for (int m = 0; m < TM * TN; ++m) {
                const int i = m / TN, j = m % TN;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], bfr[ks & 1][j], acc[i][j], 0, 0, 0);
                const int q = ks * IPK + m / MPI;
                if (m % MPI == MPI - 1 && m / MPI < IPK && q < NI) item(wa, wb, ra, rb, q, kt3);
            }
            if (ks < 3) __builtin_amdgcn_sched_group_barrier(0x100, NFR, 0);   // next fragments
#pragma unroll
            for (int g = 0; g < IPK; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x008, MPI, 0);                // MPI MFMAs
                if (ks * IPK + g < NI) {
                    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);              // 1 LDS store
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);              // 1 global load
                }
            }
            if constexpr (TM * TN > MPI * IPK)
                __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - MPI * IPK, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    u32x4 ra0[QA], rb0[QB], ra1[QA], rb1[QB];
    gload(ra0, rb0, 0);
    gload(ra1, rb1, 1);
    lstore(sA0, sB0, ra0, rb0);
    gload(ra0, rb0, 2);
    __syncthreads();
    // Slice kt reads buffer kt % 2 and stages slice kt + 1 into the other one,
    // whose last reader (slice kt - 1) finished before the previous barrier.
    // An odd slice count runs one all-zero slice at the end; the last pair
    // stages a past-the-end slice into a buffer nobody reads.
    for (int kt = 0; kt < nk; kt += 2) {
        slice(sA0, sB0, sA1, sB1, ra1, rb1, kt + 3);
        __syncthreads();
        slice(sA1, sB1, sA0, sB0, ra0, rb0, kt + 4);
        __syncthreads();
    }

    // acc[i][j][v]: row 8 (v / 4) + 4 (lane / 32) + v % 4, column lane % 32 of its 32x32 tile
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * (BN / 2) + j * 32 + r32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm * (BM / WM) + i * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
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
// dimension (a contiguous quarter of the k-steps each) and each computes a
// 16 tokens x 16 neurons partial product with v_mfma_f32_16x16x32_bf16 (A =
// tokens, rows past the batch are zero and load nothing; B = 16 rows of W).
// The partials are summed in LDS in wave order, the bias is added, and the up
// projection is then computed only for neurons with g > 0 for some token of
// the tile: lanes of inactive neurons issue no loads, so the rows of W_up of
// inactive neurons are never read.
// ---------------------------------------------------------------------------

// Each wave takes a contiguous quarter of d in stages of 128 features: per
// stage it loads 256 contiguous bytes of each of the 16 neuron rows (four
// lanes per row, 64 bytes each), writes them to its LDS tile (rows 272
// bytes apart, so both the 16-byte writes and the fragment reads below are
// free of bank conflicts) and reads the MFMA B operand from there; the x
// fragments (16 tokens, L2-resident) come straight from memory.  Three
// register stages keep the next two stages' loads in flight.  LDS instructions
// of one wave complete in order, so a stage's tile writes follow the
// previous stage's reads.
constexpr int kDreluStageK = 128;                 // features per stage
constexpr int kDreluPitch = kDreluStageK + 8;     // tile row pitch in bf16 (272 bytes)

// w_tile = the workgroup's first neuron row, n_tile = neurons of the tile that
// exist (both uniform); only rows whose bit is set in wmask are read.
__device__ __forceinline__ void drelu_partial(const uint16_t* __restrict__ x, int64_t rows,
                                              int64_t tok0, int64_t d,
                                              const uint16_t* __restrict__ w_tile, int64_t n_tile,
                                              uint32_t wmask, int wave, int lane, f32x4& acc,
                                              uint16_t* __restrict__ tile) {
    // Buffer views: loads never branch, and rows past the batch, inactive
    // neurons and k past the row end read zero.
    const int r16 = lane & 15, kg = lane >> 4;          // MFMA lanes: row / k group
    const int wr = lane >> 2, wsg = lane & 3;            // loading lanes: row / 64-byte segment
    constexpr uint32_t kOff = 0x40000000u;   // out of range for both views
    const int64_t ntok = min((int64_t)16, rows - tok0);
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x + tok0 * d), (short)0, (int)(ntok * d * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(w_tile), (short)0, (int)(n_tile * d * 2), 0x00020000);
    const bool wload = ((wmask >> wr) & 1u) != 0u;
    const int nst = (int)((d + kDreluStageK - 1) / kDreluStageK);
    const int per = (nst + 3) / 4;
    const int st0 = wave * per, st1 = min(nst, st0 + per);
    auto load = [&](u32x4* wv, u32x4* xv, int st) {
        const int64_t k0 = (int64_t)st * kDreluStageK;
        const bool in = st < st1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t kw = k0 + 32 * wsg + 8 * i;
            wv[i] = __builtin_amdgcn_raw_buffer_load_b128(
                wrs, in && wload && kw < d ? (uint32_t)((wr * d + kw) * 2) : kOff, 0, 0);
            const int64_t kx = k0 + 32 * i + 8 * kg;
            xv[i] = __builtin_amdgcn_raw_buffer_load_b128(
                xrs, in && kx < d ? (uint32_t)((r16 * d + kx) * 2) : kOff, 0, 0);
        }
    };
    auto compute = [&](const u32x4* wv, const u32x4* xv) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4*>(tile + wr * kDreluPitch + 32 * wsg + 8 * i) = wv[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 bv = *reinterpret_cast<const u32x4*>(tile + r16 * kDreluPitch + 32 * i + 8 * kg);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xv[i]), as_bf16x8(bv), acc, 0, 0, 0);
        }
    };
    u32x4 wa[4], xa[4], wb[4], xb[4], wc[4], xc[4];
    load(wa, xa, st0);
    load(wb, xb, st0 + 1);   // past the quarter: out of range, no data moved
    for (int st = st0; st < st1; st += 3) {
        load(wc, xc, st + 2);
        __builtin_amdgcn_sched_barrier(0);
        compute(wa, xa);
        __builtin_amdgcn_sched_barrier(0);
        if (st + 1 >= st1) break;   // uniform
        load(wa, xa, st + 3);
        __builtin_amdgcn_sched_barrier(0);
        compute(wb, xb);
        __builtin_amdgcn_sched_barrier(0);
        if (st + 2 >= st1) break;
        load(wb, xb, st + 4);
        __builtin_amdgcn_sched_barrier(0);
        compute(wc, xc);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Side jobs of a gate/up launch, done first (also by workgroups that then
// find no work): workgroup 0 clears the split-K counters of the down gather,
// and all workgroups together clear the output that the down gather adds into.
// (The fields come by value: a reference to the kernel's argument struct
// costs the kernels registers.)
__device__ __forceinline__ void drelu_side_clear(int32_t* zero_ptr, int n_zero, float* zero_out,
                                                 int64_t n_zero_out, int tid) {
    if (blockIdx.x == 0 && blockIdx.y == 0 && zero_ptr != nullptr)
        for (int i = tid; i < n_zero; i += 256) zero_ptr[i] = 0;
    if (zero_out != nullptr) {   // (n_zero_out < 2^31, checked by the launchers)
        const int n4 = (int)(n_zero_out / 4), step = (int)(gridDim.x * gridDim.y) * 256;
        uint4* z = reinterpret_cast<uint4*>(zero_out);
        for (int i = (int)(blockIdx.y * gridDim.x + blockIdx.x) * 256 + tid; i < n4; i += step)
            z[i] = make_uint4(0u, 0u, 0u, 0u);
    }
}

__global__ __launch_bounds__(256) void drelu_gate_up_kernel(DreluArgs a) {
    __shared__ f32x4 s_part[4][64];
    __shared__ __attribute__((aligned(16))) uint16_t s_tile[4][16 * kDreluPitch];
    __shared__ uint32_t s_act;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, kg = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t rows = a.rows, d = a.d, ffn = a.ffn;
    const int64_t n = n0 + r16;                 // this lane's neuron (B column / D column)
    const bool n_ok = n < ffn;

    drelu_side_clear(a.zero_ptr, a.n_zero, a.zero_out, a.n_zero_out, tid);

    for (int64_t tok0 = 0; tok0 < rows; tok0 += 16) {
        // gate partials
        const int64_t n_tile = min((int64_t)16, ffn - n0);
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        drelu_partial(a.x, rows, tok0, d, a.wg + n0 * d, n_tile, 0xFFFFu, wave, lane, acc,
                      s_tile[wave]);
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
            drelu_partial(a.x, rows, tok0, d, a.wu + n0 * d, n_tile, act, wave, lane, u, s_tile[wave]);
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

// Single-token dReLU gate/up.  With one token the projections are plain
// GEMVs, so a wavefront owns NPW neurons and reads each row as whole 1 KB
// pieces (64 lanes x 16 bytes, 8 pieces for d = 4096): lane l holds x[512 i +
// 8 l .. + 7] and the weights at the same k, all of a wavefront's gate rows are
// in flight at once, and each dot product is reduced across the wavefront
// with DPP in a fixed order.  The up rows are then loaded only for neurons
// whose gate is positive (a wavefront-uniform decision).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float dot8(const u32x4& w, const u32x4& x, float acc) {
    const uint32_t wu[4] = {w.x, w.y, w.z, w.w}, xu[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc = fmaf(__uint_as_float(wu[i] << 16), __uint_as_float(xu[i] << 16), acc);
        acc = fmaf(__uint_as_float(wu[i] & 0xFFFF0000u), __uint_as_float(xu[i] & 0xFFFF0000u), acc);
    }
    return acc;
}

template <int NCH, int NPW>
__global__ __launch_bounds__(256) void drelu_gate_up_b1_kernel(DreluArgs a) {
    // NPW neurons per wavefront
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t d = a.d, ffn = a.ffn;
    const int64_t nb = ((int64_t)blockIdx.x * 4 + wave) * NPW;
    drelu_side_clear(a.zero_ptr, a.n_zero, a.zero_out, a.n_zero_out, tid);
    // Launch row blockIdx.y: the token itself, or a (token, expert) pair.
    const int64_t pr = blockIdx.y;
    int64_t tok = 0, ex = 0;
    if (a.pair_expert != nullptr) {
        tok = a.pair_token[pr];
        ex = a.pair_expert[pr];
    }
    const uint16_t* xrow = a.x + tok * d;
    const uint16_t* wgx = a.wg + ex * ffn * d;
    const uint16_t* wux = a.wu + ex * ffn * d;
    const float* bgx = a.bg != nullptr ? a.bg + ex * ffn : nullptr;
    const float* bux = a.bu != nullptr ? a.bu + ex * ffn : nullptr;
    float* hrow = a.h + pr * ffn;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(xrow), (short)0, (int)(d * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(wgx), (short)0, (int)(ffn * d * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t ur = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(wux), (short)0, (int)(ffn * d * 2), 0x00020000);
    constexpr uint32_t kOff = 0x80000000u;
    u32x4 xv[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int64_t k = (int64_t)i * 512 + 8 * lane;
        xv[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, k < d ? (uint32_t)(k * 2) : kOff, 0, 0);
    }
    auto row_off = [&](int64_t n, int i) -> uint32_t {
        const int64_t k = (int64_t)i * 512 + 8 * lane;
        return (n < ffn && k < d) ? (uint32_t)((n * d + k) * 2) : kOff;
    };
    u32x4 wv[NPW][NCH];
#pragma unroll
    for (int j = 0; j < NPW; ++j)
#pragma unroll
        for (int i = 0; i < NCH; ++i) wv[j][i] = __builtin_amdgcn_raw_buffer_load_b128(gr, row_off(nb + j, i), 0, 0);
    float g[NPW];
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) s = dot8(wv[j][i], xv[i], s);
        g[j] = wave_sum(s) + ((bgx != nullptr && nb + j < ffn) ? bgx[nb + j] : 0.0f);
    }
    // Up rows only where the gate is positive (g is wavefront-uniform).
#pragma unroll
    for (int j = 0; j < NPW; ++j)
        if (g[j] > 0.0f)
#pragma unroll
            for (int i = 0; i < NCH; ++i) wv[j][i] = __builtin_amdgcn_raw_buffer_load_b128(ur, row_off(nb + j, i), 0, 0);
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
        float hv = 0.0f;
        if (g[j] > 0.0f) {
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < NCH; ++i) s = dot8(wv[j][i], xv[i], s);
            const float uv = wave_sum(s) + ((bux != nullptr && nb + j < ffn) ? bux[nb + j] : 0.0f);
            hv = uv > 0.0f ? __fmul_rn(g[j], uv) : 0.0f;
        }
        if (lane == 0 && nb + j < ffn) hrow[nb + j] = hv;
    }
}

// Grouped MoE gate/up: workgroup (x, y) owns neurons 8x .. 8x + 7 of expert
// y and runs them for every token routed to that expert, TC tokens at a time.
// Per chunk the workgroup stages the TC token rows of x in LDS (rows past the
// chunk are zero), then each wavefront loads its two gate rows (16-byte
// slices per lane, as in the one-token kernel); the up rows are read only for
// neurons whose gate is positive for some token of the chunk.  Each (neuron,
// token) value is the same sum in the same order as in the one-token kernel,
// so h does not depend on how the tokens are grouped.  Without expert lists
// (grp_count null) the grid has one expert and token t is row t: the dense
// dReLU FFN for a few tokens.
template <int NCH>
__global__ __launch_bounds__(256) void drelu_grouped_kernel(DreluArgs a) {
    constexpr int NPW = 2, TC = NCH <= 8 ? 4 : 2, RL = NCH * 512;   // RL: staged row length
    __shared__ __attribute__((aligned(16))) uint16_t s_x[TC][RL];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t d = a.d, ffn = a.ffn;
    const int ex = blockIdx.y;
    drelu_side_clear(a.zero_ptr, a.n_zero, a.zero_out, a.n_zero_out, tid);
    // Without expert lists (a dense FFN): one matrix, row t of x is h row t.
    const bool ident = a.grp_count == nullptr;
    const int32_t* gq = ident ? nullptr : a.grp_pairs + ex * a.pairs;
    const int32_t* gt = ident ? nullptr : a.grp_tok + ex * a.pairs;
    const int cnt = ident ? (int)a.rows : a.grp_count[ex];
    if (cnt == 0) return;   // uniform: no token chose this expert
    const int64_t nb = ((int64_t)blockIdx.x * 4 + wave) * NPW;
    const uint16_t* wgx = a.wg + ex * ffn * d;
    const uint16_t* wux = a.wu + ex * ffn * d;
    const float* bgx = a.bg != nullptr ? a.bg + ex * ffn : nullptr;
    const float* bux = a.bu != nullptr ? a.bu + ex * ffn : nullptr;
    constexpr uint32_t kOff = 0x80000000u;   // x and each expert matrix are below 2 GiB
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.x), (short)0, (int)(a.rows * d * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(wgx), (short)0, (int)(ffn * d * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t ur = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(wux), (short)0, (int)(ffn * d * 2), 0x00020000);
    auto row_off = [&](int64_t n, int i) -> uint32_t {
        const int64_t k = (int64_t)i * 512 + 8 * lane;
        return (n < ffn && k < d) ? (uint32_t)((n * d + k) * 2) : kOff;
    };
    auto xs = [&](int t, int i) {   // this lane's 8 features of run i of staged token t
        return *reinterpret_cast<const u32x4*>(&s_x[t][i * 512 + 8 * lane]);
    };
    float bg[NPW], bu[NPW];
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
        bg[j] = (bgx != nullptr && nb + j < ffn) ? bgx[nb + j] : 0.0f;
        bu[j] = (bux != nullptr && nb + j < ffn) ? bux[nb + j] : 0.0f;
    }
    constexpr int XPT = TC * RL / 8 / 256;   // 16-byte pieces of x staged per thread
    for (int c0 = 0; c0 < cnt; c0 += TC) {
        int32_t q[TC];
        int64_t tokoff[TC];   // byte offset of each token's x row (uniform)
#pragma unroll
        for (int t = 0; t < TC; ++t) {
            const bool tv = c0 + t < cnt;
            q[t] = tv ? (ident ? c0 + t : gq[c0 + t]) : -1;
            tokoff[t] = tv ? (int64_t)(ident ? c0 + t : gt[c0 + t]) * d * 2 : -1;
        }
        u32x4 xp[XPT];
#pragma unroll
        for (int r = 0; r < XPT; ++r) {
            const int ci = tid + 256 * r;
            const int t = ci / (RL / 8);   // uniform per r: RL / 8 is a multiple of 256
            const int64_t k = (int64_t)(ci % (RL / 8)) * 8;
            xp[r] = __builtin_amdgcn_raw_buffer_load_b128(
                xr, (tokoff[t] >= 0 && k < d) ? (uint32_t)(tokoff[t] + k * 2) : kOff, 0, 0);
        }
        __syncthreads();   // the previous chunk's reads of s_x are done
#pragma unroll
        for (int r = 0; r < XPT; ++r) {
            const int ci = tid + 256 * r;
            *reinterpret_cast<u32x4*>(&s_x[ci / (RL / 8)][(ci % (RL / 8)) * 8]) = xp[r];
        }
        // The gate rows are loaded after the (short, L2-resident) x staging,
        // so that the staging registers are free again while they are in flight.
        u32x4 wv[NPW][NCH];
#pragma unroll
        for (int j = 0; j < NPW; ++j)
#pragma unroll
            for (int i = 0; i < NCH; ++i) wv[j][i] = __builtin_amdgcn_raw_buffer_load_b128(gr, row_off(nb + j, i), 0, 0);
        __syncthreads();
        // Token by token, so that only one token's slices are held (the
        // scheduling barriers keep the LDS reads of the next token from
        // being hoisted).  The empty asm statements mark the packed weights
        // and slices as changed per token and neuron, so that their unpacked
        // fp32 values (twice the registers) are not kept for reuse.
        float g[NPW][TC];
        bool need[NPW] = {};
#pragma unroll
        for (int t = 0; t < TC; ++t) {
#pragma unroll
            for (int j = 0; j < NPW; ++j)
#pragma unroll
                for (int i = 0; i < NCH; ++i) asm volatile("" : "+v"(wv[j][i]));
            u32x4 xt[NCH];
#pragma unroll
            for (int i = 0; i < NCH; ++i) xt[i] = xs(t, i);
#pragma unroll
            for (int j = 0; j < NPW; ++j) {
#pragma unroll
                for (int i = 0; i < NCH; ++i) asm volatile("" : "+v"(xt[i]));   // unpack per neuron
                float s = 0.0f;
#pragma unroll
                for (int i = 0; i < NCH; ++i) s = dot8(wv[j][i], xt[i], s);
                g[j][t] = wave_sum(s) + bg[j];
                need[j] = need[j] || (q[t] >= 0 && g[j][t] > 0.0f);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // Up rows only where some token's gate is positive: the other lanes'
        // offsets are out of range, so those loads move no data (and the
        // gate rows are dead from here, whatever the branch).
        u32x4 uw[NPW][NCH];
#pragma unroll
        for (int j = 0; j < NPW; ++j)
#pragma unroll
            for (int i = 0; i < NCH; ++i)
                uw[j][i] = __builtin_amdgcn_raw_buffer_load_b128(ur, need[j] ? row_off(nb + j, i) : kOff, 0, 0);
#pragma unroll
        for (int t = 0; t < TC; ++t) {
#pragma unroll
            for (int j = 0; j < NPW; ++j)
#pragma unroll
                for (int i = 0; i < NCH; ++i) asm volatile("" : "+v"(uw[j][i]));
            u32x4 xt[NCH];
#pragma unroll
            for (int i = 0; i < NCH; ++i) xt[i] = xs(t, i);
#pragma unroll
            for (int j = 0; j < NPW; ++j) {
                float hv = 0.0f;
                if (need[j] && q[t] >= 0 && g[j][t] > 0.0f) {
#pragma unroll
                    for (int i = 0; i < NCH; ++i) asm volatile("" : "+v"(xt[i]));
                    float s = 0.0f;
#pragma unroll
                    for (int i = 0; i < NCH; ++i) s = dot8(uw[j][i], xt[i], s);
                    const float uv = wave_sum(s) + bu[j];
                    hv = uv > 0.0f ? __fmul_rn(g[j][t], uv) : 0.0f;
                }
                if (lane == 0 && q[t] >= 0 && nb + j < ffn) a.h[(int64_t)q[t] * ffn + nb + j] = hv;
            }
            __builtin_amdgcn_sched_barrier(0);
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

template <int BN, int NW, bool AK, bool BK>
hipError_t launch_gemm_deep(const uint16_t* A, const uint16_t* B, void* C, int64_t m, int64_t n,
                            int64_t k, int64_t lda, int64_t ldb, int c_bf16, hipStream_t stream) {
    const int tiles_m = (int)((m + 255) / 256), tiles_n = (int)((n + BN - 1) / BN);
    gemm_bf16_deep_kernel<BN, NW, AK, BK><<<dim3(tiles_m * tiles_n), dim3(64 * NW), 0, stream>>>(
        A, B, C, (int)m, (int)n, (int)k, (int)lda, (int)ldb, c_bf16, tiles_m, tiles_n);
    return hipGetLastError();
}

// Idle share of the last round of workgroups (one 256 x BN tile per CU).
double tile_waste(int64_t m, int64_t n, int bn) {
    const int64_t t = (m + 255) / 256 * ((n + bn - 1) / bn);
    const int64_t r = (t + 255) / 256 * 256;
    return (double)(r - t) / (double)r;
}

template <bool AK, bool BK>
hipError_t launch_gemm_layout(const GemmArgs& g, hipStream_t stream) {
    // (k-contiguous A, k-major B) at BN = 192 would need more than the 256
    // registers a wavefront has at two wavefronts per SIMD: 128 only.
    if ((!AK && BK) || tile_waste(g.m, g.n, 128) + 1e-9 < tile_waste(g.m, g.n, 192))
        return launch_gemm_deep<128, 8, AK, BK>(g.a, g.b, g.c, g.m, g.n, g.k, g.lda, g.ldb, g.c_bf16, stream);
    if constexpr (!AK && BK) return hipErrorInvalidValue;   // not reached
    else return launch_gemm_deep<192, 8, AK, BK>(g.a, g.b, g.c, g.m, g.n, g.k, g.lda, g.ldb, g.c_bf16, stream);
}

}  // namespace

hipError_t launch_masked_gemm(const MfmaArgs& a, hipStream_t stream) {
    if (a.m <= 0 || a.n <= 0) return hipSuccess;
    // Pick the tile width that leaves the fewest idle workgroup slots on 256 CUs.
    const int64_t tm = (a.m + 255) / 256;
    const int64_t t256 = tm * ((a.n + 255) / 256), t192 = tm * ((a.n + 191) / 192);
    auto waste = [](int64_t t) { int64_t r = (t + 255) / 256 * 256; return (double)(r - t) / r; };
    const bool w192 = waste(t192) + 1e-9 < waste(t256);
    if (a.k % 128 == 0 && (int64_t)a.m * a.k < (int64_t(1) << 30) && (int64_t)a.n * a.k < (int64_t(1) << 30))
        return launch_gemm_deep<192, 8, false, false>(a.x, a.w, a.y, a.m, a.n, a.k, a.k, a.k, a.y_bf16, stream);
    if (w192) return launch_gemm_cfg<256, 192, 2, 3>(a, stream);
    return launch_gemm_cfg<256, 256, 2, 4>(a, stream);
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t stream) {
    if (g.m <= 0 || g.n <= 0) return hipSuccess;
    if (!g.a_kmajor && !g.b_kmajor) return launch_gemm_layout<false, false>(g, stream);
    if (!g.a_kmajor && g.b_kmajor) return launch_gemm_layout<false, true>(g, stream);
    if (g.a_kmajor && g.b_kmajor) return launch_gemm_layout<true, true>(g, stream);
    return hipErrorInvalidValue;   // k-major A with k-contiguous B: not instantiated
}

hipError_t launch_drelu_gate_up(const DreluArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    if (a.zero_out != nullptr && (a.n_zero_out % 4 != 0 || a.n_zero_out >= (int64_t(1) << 31)))
        return hipErrorInvalidValue;
    const unsigned blocks = (unsigned)((a.ffn + 15) / 16);
    const bool moe = a.pair_expert != nullptr;
    if (moe && a.d > 8192) return hipErrorInvalidValue;
    if ((a.rows == 1 || moe) && a.d <= 8192) {   // two neurons per wavefront, eight per workgroup
        const int nch = (int)((a.d + 511) / 512);
        const dim3 g2((unsigned)((a.ffn + 7) / 8), moe ? (unsigned)a.pairs : 1u);
        if (nch <= 4) drelu_gate_up_b1_kernel<4, 2><<<g2, dim3(256), 0, stream>>>(a);
        else if (nch <= 8) drelu_gate_up_b1_kernel<8, 2><<<g2, dim3(256), 0, stream>>>(a);
        else drelu_gate_up_b1_kernel<16, 2><<<g2, dim3(256), 0, stream>>>(a);
        return hipGetLastError();
    }
    if (a.rows <= 4 && a.d <= 8192) {
        // One chunk of the grouped kernel (every token, one matrix) streams the
        // gate faster than 16-token MFMA tiles: 49 / 60 us for the Mistral-7B
        // FFN at 2 / 4 tokens against 54 / 68.  With more chunks it re-reads
        // the gate rows once the L2 has dropped them.
        DreluArgs b = a;
        b.n_experts = 1;
        b.grp_count = nullptr;
        return launch_drelu_grouped(b, stream);
    }
    drelu_gate_up_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_drelu_grouped(const DreluArgs& a, hipStream_t stream) {
    if (a.rows <= 0 || (a.grp_count != nullptr && a.pairs <= 0)) return hipSuccess;
    if (a.zero_out != nullptr && (a.n_zero_out % 4 != 0 || a.n_zero_out >= (int64_t(1) << 31)))
        return hipErrorInvalidValue;
    if (a.d > 8192 || a.n_experts < 1 || a.n_experts > 64 ||
        a.rows * a.d * 2 >= (int64_t(1) << 31) || a.ffn * a.d * 2 >= (int64_t(1) << 31))
        return hipErrorInvalidValue;
    const int nch = (int)((a.d + 511) / 512);
    const dim3 grid((unsigned)((a.ffn + 7) / 8), (unsigned)a.n_experts);
    if (nch <= 4) drelu_grouped_kernel<4><<<grid, dim3(256), 0, stream>>>(a);
    else if (nch <= 8) drelu_grouped_kernel<8><<<grid, dim3(256), 0, stream>>>(a);
    else drelu_grouped_kernel<16><<<grid, dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_nonzero_lists(const float* h, int64_t rows, int64_t n, int32_t* idx,
                                int32_t* cnt, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    nonzero_lists_kernel<<<dim3((unsigned)rows), dim3(256), 0, stream>>>(h, n, idx, cnt);
    return hipGetLastError();
}

}  // namespace qs
