// Block Q-Sparse on gfx950's structured-sparse matrix cores.
//
// Q-Sparse abstract (arXiv 2407.10969 listing page) introduces Block
// Q-Sparse for batch training and inference; the page's Chinese summary
// (method details, key-design item 3) adds only that the activations are
// split into blocks to use the hardware better.  The rule is not given; the
// reading implemented here is the Top-K section's top-K taken inside every
// contiguous block of 4 features of a token, keeping 2 (ties to the lower
// index): the 2:4 pattern that v_smfmac_f32_32x32x32_bf16 consumes, so the
// batched product Y = (X (.) M) . W^T runs at the sparse rate.
//
// Operand layout of v_smfmac_f32_32x32x32_bf16 (measured on the device with
// one-hot inputs and checked on random ones):
//   A (sparse, 32 x 32): lane l holds row l % 32; with kg = l / 32 its 8
//     values are 2 per 4-feature group g = 0..3, the groups covering features
//     16 (g / 2) + 8 kg + 4 (g % 2) + {0..3} of the 32; value e sits at the
//     position held in index bits [2e + 1 : 2e] (the low 16 bits of the index
//     operand with abid = 0);
//   B (dense, 32 x 32): lane l holds column l % 32, features 16 (l / 32) + e,
//     e = 0..15;
//   D: as v_mfma_f32_32x32x16: lane l, value v -> row 8 (v / 4) + 4 (l / 32)
//     + v % 4, column l % 32.
#include "qs_internal.h"

namespace qs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

// ---------------------------------------------------------------------------
// 2:4 selection and packing.  The packed operand is slice-major (a slice is
// 64 features = two 32-feature k-blocks):
//   av  [nslices][rows][4] 16-byte chunks: chunk 2 kb + kg holds the 8 kept
//       values of k-block kb that lane half kg of the sparse MFMA reads
//       (4-feature groups 2kg, 2kg+1, 4+2kg, 5+2kg of the k-block, two values
//       each in ascending position);
//   ai  [nslices][rp][4] u16 (rp = rows rounded up to even, so that a slice
//       plane is a whole number of 16-byte chunks of two rows): entry
//       2 kb + kg is that lane half's index
//       bits (group g in bits 4g..4g+3: first position | second << 2), so
//       the u32 at [.., kb] is the index word of k-block kb with kg = 0 in
//       the low half.
// One thread per (row, slice, kb, kg): it reads two runs of 8 features
// (8 kg .. 8 kg + 7 and 16 + 8 kg .. of the k-block).  K-blocks past d are
// written as zeros with positions (0, 1).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void nm24_pack_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t d, int64_t nslices,
    u32x4* __restrict__ av, uint16_t* __restrict__ ai, uint8_t* __restrict__ mask) {
    const int64_t rp = rows + (rows & 1);
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t units = rows * nslices * 4;
    if (t >= units) return;
    const int kg = (int)(t & 1), kb = (int)((t >> 1) & 1);
    const int64_t rs = t >> 2;                 // row * nslices + slice
    const int64_t s = rs % nslices, r = rs / nslices;
    const int64_t f0 = s * 64 + 32 * kb;       // first feature of the k-block
    uint16_t v[8];
    uint32_t bits = 0;
    uint8_t mk[16];
    if (f0 < d) {
        const u32x4* src = reinterpret_cast<const u32x4*>(x + r * d + f0);
        const u32x4 run0 = src[kg], run1 = src[2 + kg];
        uint16_t e[16];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            e[2 * w] = (uint16_t)(run0[w] & 0xFFFFu);
            e[2 * w + 1] = (uint16_t)(run0[w] >> 16);
            e[8 + 2 * w] = (uint16_t)(run1[w] & 0xFFFFu);
            e[8 + 2 * w + 1] = (uint16_t)(run1[w] >> 16);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint32_t key[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) key[i] = e[4 * g + i] & 0x7FFFu;
            int n = 0, pos[2] = {0, 1};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int rank = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    rank += (key[j] > key[i]) || (key[j] == key[i] && j < i);
                const bool keep = rank < 2;
                mk[4 * g + i] = keep;
                if (keep) {
                    if (n == 0) pos[0] = i; else pos[1] = i;
                    ++n;
                }
            }
            v[2 * g] = e[4 * g + pos[0]];
            v[2 * g + 1] = e[4 * g + pos[1]];
            bits |= (uint32_t)(pos[0] | (pos[1] << 2)) << (4 * g);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) mk[i] = 0;
        bits = 0x4444u;
    }
    u32x4 pk;
#pragma unroll
    for (int w = 0; w < 4; ++w) pk[w] = (uint32_t)v[2 * w] | ((uint32_t)v[2 * w + 1] << 16);
    av[(s * rows + r) * 4 + 2 * kb + kg] = pk;
    ai[(s * rp + r) * 4 + 2 * kb + kg] = (uint16_t)bits;
    if (mask && f0 < d) {
        uint8_t* m = mask + r * d + f0;
        uint64_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            lo |= (uint64_t)mk[i] << (8 * i);
            hi |= (uint64_t)mk[8 + i] << (8 * i);
        }
        *reinterpret_cast<uint64_t*>(m + 8 * kg) = lo;
        *reinterpret_cast<uint64_t*>(m + 16 + 8 * kg) = hi;
    }
}

// ---------------------------------------------------------------------------
// Y[M, N] = A . W^T with A the packed 2:4 operand (M = tokens, K = features)
// and W [N, K] bf16 (nn.Linear layout).  Tile 256 x BN x 64 per workgroup of
// NW wavefronts (NW / 2 x 2, each 256 / (NW / 2) x BN / 2, 32 x 32 MFMA
// tiles); two sparse k-steps of 32 per slice.  Staging as in the dense deep
// GEMM: slices go global -> registers two ahead and registers -> LDS (double
// buffer) one ahead, one barrier per slice, each chunk's LDS store and
// register reload interleaved with the MFMAs.
// LDS: values 4 chunks per row at position c ^ ((row >> 2) & 3) (16 rows of
// one pass hit 16 distinct 16-byte bank groups); index words 2 per row; W
// rows 8 chunks at c ^ ((row >> 1) & 7) as in the dense kernel.
// ---------------------------------------------------------------------------
template <int BN, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_sp24_kernel(
    const u32x4* __restrict__ av, const uint32_t* __restrict__ ai,
    const uint16_t* __restrict__ W, void* __restrict__ C,
    int M, int N, int K, int nslices, int c_bf16, int tiles_m, int tiles_n) {
    constexpr int NTH = 64 * NW, WM = NW / 2;
    constexpr int BM = 256, TM = BM / WM / 32, TN = BN / 64;
    constexpr int QA = BM * 4 / NTH;           // value chunks per thread per slice
    constexpr int QB = BN * 8 / NTH;           // W chunks per thread per slice
    constexpr int NIDX = BM * 8 / 16;          // index chunks per slice (threads < NIDX load one)
    static_assert(BN % 64 == 0 && (BM * 4) % NTH == 0 && (BN * 8) % NTH == 0 && NIDX <= NTH, "tile");
    __shared__ u32x4 sV0[BM * 4], sV1[BM * 4];
    __shared__ u32x4 sI0[NIDX], sI1[NIDX];
    __shared__ u32x4 sB0[BN * 8], sB1[BN * 8];

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

    // Value chunk q: slot sl = q * NTH + tid -> row sl / 4, chunk sl % 4 (rows
    // past M repeat the last row; never stored).  Offsets in 16-byte units
    // within a slice plane of M rows; the plane advances by 4 M per slice.
    int offv[QA], offw[QB];
#pragma unroll
    for (int q = 0; q < QA; ++q) {
        const int sl = q * NTH + tid;
        offv[q] = min(m0 + (sl >> 2), M - 1) * 4 + (sl & 3);
    }
    // Index chunk of this thread (threads < NIDX): rows m0 + 2 tid and +1, in
    // 16-byte units within the index plane ((M + 1) / 2 chunks of two rows).
    const int offi = (m0 >> 1) + tid;
    const bool has_idx = tid < NIDX && m0 + 2 * tid < M;
#pragma unroll
    for (int q = 0; q < QB; ++q) {
        const int sl = q * NTH + tid, row = sl >> 3, c = (sl & 7) ^ ((row >> 1) & 7);
        offw[q] = min(n0 + row, N - 1) * K + 8 * c;
    }
    const int kcw = 8 * ((tid & 7) ^ ((tid >> 4) & 7));   // k offset of this thread's W chunks
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4*>(av), (short)0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t ir = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(ai), (short)0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(W), (short)0, 0x7FFFFFFF, 0x00020000);
    // The index plane of a slice holds (M + 1) / 2 chunks (two rows each).
    const uint32_t iplane = (uint32_t)((M + 1) / 2);
    auto voff = [&](int q, int kt) -> uint32_t {
        return kt < nslices ? ((uint32_t)kt * 4u * (uint32_t)M + (uint32_t)offv[q]) * 16u : 0x80000000u;
    };
    auto ioff = [&](int kt) -> uint32_t {
        return (kt < nslices && has_idx) ? ((uint32_t)kt * iplane + (uint32_t)offi) * 16u : 0x80000000u;
    };
    auto woff = [&](int q, int kt) -> uint32_t {
        return 64 * kt + kcw < K ? ((uint32_t)offw[q] + 64u * (uint32_t)kt) * 2u : 0x80000000u;
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int r32 = lane & 31, kg = lane >> 5;
    auto frag = [&](const u32x4* sv, const u32x4* si, const u32x4* sb, int ks, bf16x8* af,
                    uint32_t* ix, bf16x16* bfr) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm * (BM / WM) + i * 32 + r32;
            af[i] = __builtin_bit_cast(bf16x8, sv[row * 4 + ((2 * ks + kg) ^ ((row >> 2) & 3))]);
            ix[i] = reinterpret_cast<const uint32_t*>(si)[row * 2 + ks] >> (16 * kg);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int row = wn * (BN / 2) + j * 32 + r32, sw = (row >> 1) & 7, c = 4 * ks + 2 * kg;
            const u32x4 lo = sb[row * 8 + (c ^ sw)], hi = sb[row * 8 + ((c + 1) ^ sw)];
            bfr[j] = __builtin_bit_cast(bf16x16, u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        }
    };
    // Staging items per slice: QA value chunks, one index chunk, QB W chunks.
    constexpr int NI = QA + 1 + QB;
    constexpr int IPK = (NI + 1) / 2;          // items per k-step (two k-steps per slice)
    constexpr int MPI = (TM * TN) / IPK;       // MFMAs before each item
    static_assert(MPI >= 1 && 2 * IPK >= NI, "staging schedule");
    constexpr int NFR = 2 * TM + 2 * TN;       // LDS reads per k-step
    auto lslot = [&](int q) -> int { const int sl = q * NTH + tid; return (sl >> 2) * 4 + ((sl & 3) ^ (((sl >> 2) >> 2) & 3)); };
    auto item = [&](u32x4* wv, u32x4* wi, u32x4* wb, u32x4* rv, u32x4& ri, u32x4* rb, int q, int kt3) {
        if (q < QA) {
            wv[lslot(q)] = rv[q];
            rv[q] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff(q, kt3), 0, 0);
        } else if (q == QA) {
            if (tid < NIDX) wi[tid] = ri;
            ri = __builtin_amdgcn_raw_buffer_load_b128(ir, ioff(kt3), 0, 0);
        } else {
            const int qb = q - QA - 1;
            wb[qb * NTH + tid] = rb[qb];
            rb[qb] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff(qb, kt3), 0, 0);
        }
    };
    auto gload = [&](u32x4* rv, u32x4& ri, u32x4* rb, int kt) {
#pragma unroll
        for (int q = 0; q < QA; ++q) rv[q] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff(q, kt), 0, 0);
        ri = __builtin_amdgcn_raw_buffer_load_b128(ir, ioff(kt), 0, 0);
#pragma unroll
        for (int q = 0; q < QB; ++q) rb[q] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff(q, kt), 0, 0);
    };
    auto lstore = [&](u32x4* sv, u32x4* si, u32x4* sb, const u32x4* rv, const u32x4& ri, const u32x4* rb) {
#pragma unroll
        for (int q = 0; q < QA; ++q) sv[lslot(q)] = rv[q];
        if (tid < NIDX) si[tid] = ri;
#pragma unroll
        for (int q = 0; q < QB; ++q) sb[q * NTH + tid] = rb[q];
    };
    auto slice = [&](const u32x4* sv, const u32x4* si, const u32x4* sb, u32x4* wv, u32x4* wi,
                     u32x4* wb, u32x4* rv, u32x4& ri, u32x4* rb, int kt3) {
        bf16x8 af[2][TM];
        uint32_t ix[2][TM];
        bf16x16 bfr[2][TN];
        frag(sv, si, sb, 0, af[0], ix[0], bfr[0]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (ks < 1) frag(sv, si, sb, 1, af[1], ix[1], bfr[1]);
#pragma unroll
            for (int m = 0; m < TM * TN; ++m) {
                const int i = m / TN, j = m % TN;
                acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(af[ks][i], bfr[ks][j], acc[i][j],
                                                                      (int)ix[ks][i], 0, 0);
                const int q = ks * IPK + m / MPI;
                if (m % MPI == MPI - 1 && m / MPI < IPK && q < NI) item(wv, wi, wb, rv, ri, rb, q, kt3);
            }
            if (ks < 1) __builtin_amdgcn_sched_group_barrier(0x100, NFR, 0);   // next fragments
#pragma unroll
            for (int g = 0; g < IPK; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x008, MPI, 0);
                if (ks * IPK + g < NI) {
                    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
            }
            if constexpr (TM * TN > MPI * IPK)
                __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - MPI * IPK, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    u32x4 rv0[QA], rb0[QB], rv1[QA], rb1[QB], ri0, ri1;
    gload(rv0, ri0, rb0, 0);
    gload(rv1, ri1, rb1, 1);
    lstore(sV0, sI0, sB0, rv0, ri0, rb0);
    gload(rv0, ri0, rb0, 2);
    __syncthreads();
    for (int kt = 0; kt < nslices; kt += 2) {
        slice(sV0, sI0, sB0, sV1, sI1, sB1, rv1, ri1, rb1, kt + 3);
        __syncthreads();
        slice(sV1, sI1, sB1, sV0, sI0, sB0, rv0, ri0, rb0, kt + 4);
        __syncthreads();
    }

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

}  // namespace

size_t nm24_packed_bytes(int64_t rows, int64_t d) {
    const int64_t ns = (d + 63) / 64;
    const size_t vbytes = (size_t)ns * (size_t)rows * 64;
    const size_t ibytes = (size_t)ns * (size_t)((rows + 1) / 2) * 16;
    return ((vbytes + 255) & ~size_t(255)) + ((ibytes + 255) & ~size_t(255));
}

hipError_t launch_block_sparse_linear(const BlockSparseArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    const int64_t ns = (a.d + 63) / 64;
    const size_t vbytes = ((size_t)ns * (size_t)a.rows * 64 + 255) & ~size_t(255);
    u32x4* av = reinterpret_cast<u32x4*>(a.ws);
    uint32_t* ai = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(a.ws) + vbytes);
    // Index plane of a slice: (rows + 1) / 2 chunks of two rows (8 bytes a
    // row); an odd row count leaves the plane's last 8 bytes unwritten (they
    // pair with a row past M, whose results are never stored).
    const int64_t units = a.rows * ns * 4;
    nm24_pack_kernel<<<dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream>>>(
        a.x, a.rows, a.d, ns, av, reinterpret_cast<uint16_t*>(ai), a.mask);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int BN = 192;
    const int tiles_m = (int)((a.rows + 255) / 256), tiles_n = (int)((a.n + BN - 1) / BN);
    gemm_sp24_kernel<BN, 8><<<dim3(tiles_m * tiles_n), dim3(512), 0, stream>>>(
        av, ai, a.w, a.y, (int)a.rows, (int)a.n, (int)a.d, (int)ns, a.y_bf16, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace qs
