// Helpers of the kernels that take a top-K selection as a descriptor.
//
// Q-Sparse news article (zxwl-tech.com), section "Sparsification with the
// Top-K function": keep the K entries of largest |x|; ties (not covered by
// the pages) go to the lower index.  The descriptor (tau, cutoff) fixes the
// selected set: entry j is selected iff key_j > tau, or key_j == tau and
// j < cutoff, with key_j the magnitude bit pattern of entry j.
#pragma once
#include "qs_select.h"

namespace qs {
namespace rowsel {

// Exclusive prefix over the threads of a workgroup (in thread order) of one
// count per thread; `tot` receives the total.  Two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, int tid,
                                                    uint32_t& tot) {
    constexpr int NW = NT / sel::kWave;
    const int lane = tid & (sel::kWave - 1), wave = tid / sel::kWave;
    const uint32_t inc = sel::wave_incl_scan_dpp(v);
    if (lane == sel::kWave - 1) wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0, t = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t c = wsum[w];
        before += w < wave ? c : 0u;
        t += c;
    }
    __syncthreads();   // wsum may be reused after this
    tot = t;
    return before + inc - v;
}

// Per-thread selection masks of the top-k of 15-bit keys (bf16 magnitudes)
// held by a workgroup in contiguous runs (thread t holds entries
// [t E, t E + E); kInvalid past the row end), for up to BT rows at once:
//   level 1: an LDS histogram of the 8 high key bits (256 bins, in four
//            copies to spread the atomics on an activation's few exponents); every
//            wavefront reads it from the top (4 bins per lane, one DPP scan)
//            and finds the bin of the k-th largest key and its rank there;
//   level 2: a histogram of the 7 low bits of the keys in that bin (128
//            bins), read the same way: tau, how many keys equal to it are
//            taken and how many there are;
//   ties:    only when some keys equal to tau stay out, a block prefix count
//            of them in index order lets each thread take its own.
// Three or four barriers, no broadcast of the result.  L must be zeroed, and
// a barrier passed, before the call.
template <int BT, int NW>
struct Sel15Lds {
    uint32_t h1[BT][4][256];   // four copies (by lane % 4): the few exponent bins of
                               // an activation would serialise one copy's atomics
    uint32_t h2[BT][128];
    uint32_t tie[BT][NW];
};

template <int NT, int BT, int E>
__device__ __forceinline__ void select15_masks(const uint32_t (&key)[BT][E], int ntok, int64_t k,
                                               Sel15Lds<BT, NT / 64>& L, int tid,
                                               uint32_t (&selm)[BT]) {
    constexpr int NW = NT / 64;
    const int lane = tid & 63, wave = tid / 64;
    const uint32_t kk = (uint32_t)k;
#pragma unroll
    for (int t = 0; t < BT; ++t) {
        if (t >= ntok) break;
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (key[t][e] != sel::kInvalid) atomicAdd(&L.h1[t][lane & 3][key[t][e] >> 7], 1u);
    }
    __syncthreads();
    uint32_t b1[BT], r1[BT];
#pragma unroll
    for (int t = 0; t < BT; ++t) {
        b1[t] = 0xFFFFFFFFu; r1[t] = 0;
        if (t >= ntok || kk == 0) continue;   // uniform
        uint32_t c[4], sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = 255 - 4 * lane - i;
            c[i] = L.h1[t][0][b] + L.h1[t][1][b] + L.h1[t][2][b] + L.h1[t][3][b];
            sum += c[i];
        }
        const uint32_t incl = sel::wave_incl_scan_dpp(sum);
        uint32_t e = incl - sum, bin = 0, rank = 0;
        bool found = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!found && e < kk && kk <= e + c[i]) { found = true; bin = 255u - 4u * lane - i; rank = kk - e; }
            e += c[i];
        }
        const uint64_t hit = __ballot(found);
        const int src = (int)__builtin_ctzll(hit);
        b1[t] = (uint32_t)__builtin_amdgcn_readlane((int)bin, src);
        r1[t] = (uint32_t)__builtin_amdgcn_readlane((int)rank, src);
#pragma unroll
        for (int e2 = 0; e2 < E; ++e2)
            if (key[t][e2] != sel::kInvalid && (key[t][e2] >> 7) == b1[t])
                atomicAdd(&L.h2[t][key[t][e2] & 127u], 1u);
    }
    __syncthreads();
    uint32_t tau[BT], need[BT];
    bool ties = false;
#pragma unroll
    for (int t = 0; t < BT; ++t) {
        tau[t] = 0xFFFFFFFFu; need[t] = 0;
        if (t >= ntok || kk == 0) continue;   // uniform
        const uint32_t c0 = L.h2[t][127 - 2 * lane], c1 = L.h2[t][126 - 2 * lane];
        const uint32_t incl = sel::wave_incl_scan_dpp(c0 + c1);
        const uint32_t excl = incl - c0 - c1;
        const bool in0 = excl < r1[t] && r1[t] <= excl + c0;
        const bool in1 = !in0 && excl + c0 < r1[t] && r1[t] <= incl;
        const uint64_t hit = __ballot(in0 || in1);
        const int src = (int)__builtin_ctzll(hit);
        const uint32_t m = in0 ? 127u - 2u * lane : 126u - 2u * lane;
        const uint32_t nd = in0 ? r1[t] - excl : r1[t] - excl - c0;
        const uint32_t eq = in0 ? c0 : c1;
        tau[t] = (b1[t] << 7) | (uint32_t)__builtin_amdgcn_readlane((int)m, src);
        need[t] = (uint32_t)__builtin_amdgcn_readlane((int)nd, src);
        const uint32_t eqn = (uint32_t)__builtin_amdgcn_readlane((int)eq, src);
        if (need[t] < eqn) {   // uniform: some keys equal to tau stay out
            ties = true;
            uint32_t cnt = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) cnt += key[t][e] == tau[t] ? 1u : 0u;
            const uint32_t wi = sel::wave_incl_scan_dpp(cnt);
            if (lane == 63) L.tie[t][wave] = wi;
            need[t] |= 0x80000000u;   // mark: rank the ties
            r1[t] = wi - cnt;         // this thread's ties before it inside the wavefront
        }
    }
    if (ties) __syncthreads();   // uniform
#pragma unroll
    for (int t = 0; t < BT; ++t) {
        selm[t] = 0;
        if (t >= ntok || kk == 0) continue;   // uniform
        const bool rank_ties = (need[t] & 0x80000000u) != 0;
        const uint32_t nd = need[t] & 0x7FFFFFFFu;
        uint32_t r = 0;
        if (rank_ties) {
#pragma unroll
            for (int w = 0; w < NW; ++w) r += w < wave ? L.tie[t][w] : 0u;
            r += r1[t];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t kv = key[t][e];
            if (kv == sel::kInvalid) continue;
            const bool tie = kv == tau[t];
            const bool on = kv > tau[t] || (tie && (!rank_ties || r < nd));
            r += tie ? 1u : 0u;
            selm[t] |= (on ? 1u : 0u) << e;
        }
    }
}

__device__ __forceinline__ bool selected(uint32_t key, uint32_t j, uint32_t tau, uint32_t cutoff) {
    return key > tau || (key == tau && j < cutoff);
}

}  // namespace rowsel
}  // namespace qs
