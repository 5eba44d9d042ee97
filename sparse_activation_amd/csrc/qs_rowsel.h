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

__device__ __forceinline__ bool selected(uint32_t key, uint32_t j, uint32_t tau, uint32_t cutoff) {
    return key > tau || (key == tau && j < cutoff);
}

}  // namespace rowsel
}  // namespace qs
