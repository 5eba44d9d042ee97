// Device-side radix select of the K largest magnitude keys of one row held
// by a workgroup (the select step of the top-K kernel).
//
// Q-Sparse news article (zxwl-tech.com), section "Sparsification with the
// Top-K function": keep the K entries of largest |x|; among equal |x| the
// lower index wins (a reading: the pages do not cover ties).  Keys are the
// magnitude bit patterns, whose unsigned order is the order of |x|.
#pragma once
#include "qs_internal.h"

namespace qs {
namespace sel {

constexpr int kWave = 64;
constexpr uint32_t kInvalid = 0x80000000u;   // key of an entry past the row end
constexpr int kCap = 2048;                   // boundary-bin keys finished by one wavefront

__device__ __forceinline__ uint32_t popc_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive wavefront sum scan with DPP (in-register cross-lane moves:
// row_shr 1, 2, 4, 8 inside each 16-lane row, then row_bcast 15 and 31 to
// carry the row totals; out-of-row sources read zero).
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Descending search of a histogram of 64 P bins (ascending bin index = digit)
// held in LDS: lane l owns bins 64 P - 1 - P l - c (c = 0 .. P - 1).  Returns
// the digit holding the kr-th largest counted key, the rank of that key
// inside its bin and the bin count.
template <int P>
__device__ __forceinline__ void find_digit_p(const uint32_t* h, uint32_t kr, int lane,
                                             uint32_t& digit, uint32_t& kr_out, uint32_t& cnt_out) {
    static_assert(P % 4 == 0, "lanes own whole 16-byte groups of bins");
    uint32_t c[P];
#pragma unroll
    for (int g = 0; g < P / 4; ++g) {
        const uint4 v = *reinterpret_cast<const uint4*>(&h[64 * P - P * (lane + 1) + P - 4 * (g + 1)]);
        c[4 * g] = v.w; c[4 * g + 1] = v.z; c[4 * g + 2] = v.y; c[4 * g + 3] = v.x;
    }
    uint32_t lsum = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) lsum += c[i];
    const uint32_t incl = wave_incl_scan_dpp(lsum);
    const uint32_t excl = incl - lsum;
    const uint64_t bm = __ballot(excl < kr && kr <= incl);
    const int src = (int)__builtin_ctzll(bm);
    uint32_t e = excl, dg = 0, kk = 0, cn = 0;
    bool found = false;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        if (!found && e < kr && kr <= e + c[i]) {
            found = true;
            dg = (uint32_t)(64 * P - 1 - P * lane - i);
            kk = kr - e;
            cn = c[i];
        }
        e += c[i];
    }
    digit = (uint32_t)__builtin_amdgcn_readlane((int)dg, src);
    kr_out = (uint32_t)__builtin_amdgcn_readlane((int)kk, src);
    cnt_out = (uint32_t)__builtin_amdgcn_readlane((int)cn, src);
}

// Descending search over n <= 64 counts t[n - 1], ..., t[0] given in LDS:
// lane c takes t[n - 1 - c], one wave scan finds the first (from the top) whose
// running total reaches kr.  Returns its index and the total above it.
__device__ __forceinline__ void find_top_lane(const uint32_t* t, int n, uint32_t kr, int lane,
                                              int& idx, uint32_t& before) {
    const uint32_t v = lane < n ? t[n - 1 - lane] : 0u;
    const uint32_t incl = wave_incl_scan_dpp(v);
    const uint64_t bm = __ballot(incl >= kr);
    const int f = bm ? (int)__builtin_ctzll(bm) : n - 1;
    idx = n - 1 - f;
    before = (uint32_t)__builtin_amdgcn_readlane((int)(incl - v), f);
}

// LDS scratch of radix_select for keys of KB bits.  The first digit covers
// the top min(KB, 12) key bits (4096 bins, so that the few exponent values an
// activation spans spread over 16 bins each), the next ones 8 bits, every
// level with its own histogram.
// Keys of at most 20 bits (bf16, int8) have one 8-bit digit left at most, so
// they need neither the candidate list nor more than one further histogram:
// the smaller footprint lets more rows share a CU.
template <int KB>
struct SelectLds {
    static constexpr int W1 = KB < 12 ? KB : 12;
    static constexpr int S1 = KB - W1;
    static constexpr int NB1 = 1 << W1;
    static constexpr int NB1P = NB1 < 256 ? 256 : NB1;
    static constexpr int NL = S1 > 8 ? 3 : 1;          // histograms after the first digit
    static constexpr int NCAND = S1 > 8 ? kCap : 1;
    uint32_t h1[NB1P];
    uint32_t hl[NL][256];
    uint32_t cand[NCAND];
    uint32_t chunk[16];
    uint32_t res[4];
    uint32_t nc;
};

// Clear the histograms (the caller puts a barrier between this and
// radix_select).
template <int NT, int KB>
__device__ __forceinline__ void select_clear(SelectLds<KB>& s, int tid) {
    for (int i = tid; i < SelectLds<KB>::NB1P; i += NT) s.h1[i] = 0;
    for (int i = tid; i < SelectLds<KB>::NL * 256; i += NT) (&s.hl[0][0])[i] = 0;
    if (tid == 0) s.nc = 0;
}

// MSD radix select over the EPT keys each of the NT threads holds (entries
// past the row end hold kInvalid).  Returns, uniform over the workgroup, tau
// = the key of the k-th largest entry, kr = how many entries equal to tau are
// taken (those of lowest index) and eqtot = how many entries equal tau.  k >= 1.
// The digit searches run in one wavefront while the others wait at the next
// barrier: a search repeated by every wavefront costs several times over on
// each SIMD.  Zero keys (frequent: an FFN intermediate is often half zeros)
// are counted with a ballot instead of piling conflicting atomics onto bin 0.
template <int NT, int EPT, int KB>
__device__ __forceinline__ void radix_select(const uint32_t (&key)[EPT], uint32_t k,
                                             SelectLds<KB>& s, int tid, uint32_t& tau,
                                             uint32_t& kr_out, uint32_t& eqtot) {
    using L = SelectLds<KB>;
    constexpr int NW = NT / kWave, S1 = L::S1, NB1 = L::NB1;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    auto count_level = [&](uint32_t* hist, uint32_t pre, uint32_t hm, int sh, uint32_t dm) {
        uint32_t nzero = 0;   // this thread's zero keys, summed over the wavefront below
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const bool m = key[i] != kInvalid && (key[i] & hm) == pre;
            nzero += (m && key[i] == 0u) ? 1u : 0u;
            if (m && key[i] != 0u) atomicAdd(&hist[(key[i] >> sh) & dm], 1u);
        }
        nzero = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan_dpp(nzero), kWave - 1);
        if (lane == 0 && nzero != 0) atomicAdd(&hist[0], nzero);
    };
    uint32_t prefix = 0, himask = 0, kr = k, dg = 0, cnt = 0;
    count_level(s.h1, 0u, 0u, S1, (uint32_t)(NB1 - 1));
    __syncthreads();
    if constexpr (NB1 > 1024) {
        for (int c = wave; c < NB1 / 256; c += NW) {
            const uint4 v = *reinterpret_cast<const uint4*>(&s.h1[256 * c + 4 * lane]);
            const uint32_t t = wave_incl_scan_dpp(v.x + v.y + v.z + v.w);
            if (lane == kWave - 1) s.chunk[c] = t;
        }
        __syncthreads();
        if (wave == 0) {
            int cstar;
            uint32_t before;
            find_top_lane(s.chunk, NB1 / 256, kr, lane, cstar, before);
            find_digit_p<4>(s.h1 + 256 * cstar, kr - before, lane, dg, kr, cnt);
            dg += (uint32_t)(256 * cstar);
        }
    } else if (wave == 0) {
        static_assert(NB1 <= 256, "first digits of 9 to 11 bits are not used");
        find_digit_p<4>(s.h1, kr, lane, dg, kr, cnt);
    }
    if (wave == 0 && lane == 0) { s.res[0] = dg; s.res[1] = kr; s.res[2] = cnt; }
    __syncthreads();
    dg = s.res[0]; kr = s.res[1]; cnt = s.res[2];
    prefix = dg << S1;
    himask = (uint32_t)(NB1 - 1) << S1;
    // Remaining digits are 8 bits wide, each level with its own 256-bin
    // histogram hl[level], so no level clears a buffer.
    bool compact = false;
    if constexpr (S1 > 8) compact = cnt <= (uint32_t)kCap;
    if (compact) {
      if constexpr (S1 > 8) {
        // Several digits left over few keys: compact them (one LDS atomic per
        // wavefront, a wavefront prefix sum placing each thread's run; the
        // order of the candidates does not matter) and let wavefront 0
        // finish alone.
        uint32_t mc = 0;
#pragma unroll
        for (int i = 0; i < EPT; ++i)
            mc += (key[i] != kInvalid && (key[i] & himask) == prefix) ? 1u : 0u;
        const uint32_t incl = wave_incl_scan_dpp(mc);
        const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
        uint32_t base = 0;
        if (lane == 0 && wtot != 0) base = atomicAdd(&s.nc, wtot);
        uint32_t pos = (uint32_t)__builtin_amdgcn_readfirstlane((int)base) + incl - mc;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            if (key[i] != kInvalid && (key[i] & himask) == prefix) s.cand[pos++] = key[i];
        }
        __syncthreads();
        if (wave == 0 && cnt <= (uint32_t)kWave) {
            // At most one candidate per lane (the usual case: a boundary bin
            // of a 12-bit first digit holds tens of keys): every lane counts
            // the candidates above and equal to its own, broadcast one at a
            // time; the kr-th largest is a candidate c with gt(c) < kr <=
            // gt(c) + eq(c), and every lane holding that key finds the same.
            const bool have = lane < (int)cnt;
            const uint32_t c0 = s.cand[have ? lane : 0];
            uint32_t gt = 0, eq = 0;
            for (uint32_t j = 0; j < cnt; ++j) {   // uniform trip count
                const uint32_t cj = (uint32_t)__builtin_amdgcn_readlane((int)c0, (int)j);
                gt += cj > c0 ? 1u : 0u;
                eq += cj == c0 ? 1u : 0u;
            }
            const uint64_t hit = __ballot(have && gt < kr && kr <= gt + eq);
            const int src = (int)__builtin_ctzll(hit);
            const uint32_t tv = (uint32_t)__builtin_amdgcn_readlane((int)c0, src);
            const uint32_t gv = (uint32_t)__builtin_amdgcn_readlane((int)gt, src);
            const uint32_t ev = (uint32_t)__builtin_amdgcn_readlane((int)eq, src);
            if (lane == 0) { s.res[0] = tv; s.res[1] = kr - gv; s.res[2] = ev; }
        } else if (wave == 0 && cnt <= (uint32_t)(2 * kWave)) {
            // Up to two candidates per lane in wave 0's registers.
            // The remaining S1 bits are decided one at a time, most
            // significant first; the live candidates are kept as two uniform
            // ballot masks, so each bit costs one compare per register and a
            // few scalar operations.
            const uint32_t c0 = s.cand[lane < (int)cnt ? lane : 0];
            const uint32_t c1 = s.cand[lane + kWave < (int)cnt ? lane + kWave : 0];
            uint64_t live0 = __ballot(lane < (int)cnt);
            uint64_t live1 = __ballot(lane + kWave < (int)cnt);
#pragma unroll
            for (int b = S1 - 1; b >= 0; --b) {
                const uint64_t o0 = __ballot((c0 >> b) & 1u) & live0;
                const uint64_t o1 = __ballot((c1 >> b) & 1u) & live1;
                const uint32_t ones = (uint32_t)(__popcll(o0) + __popcll(o1));
                if (kr <= ones) {   // uniform
                    prefix |= 1u << b;
                    live0 = o0;
                    live1 = o1;
                } else {
                    kr -= ones;
                    live0 &= ~o0;
                    live1 &= ~o1;
                }
            }
            if (lane == 0) { s.res[0] = prefix; s.res[1] = kr; s.res[2] = (uint32_t)(__popcll(live0) + __popcll(live1)); }
        } else if (wave == 0) {
            const uint32_t ncand = cnt;
            int shift = S1, l = 0;
            while (shift > 0) {
                const int nshift = shift > 8 ? shift - 8 : 0;
                const uint32_t dmask = (1u << (shift - nshift)) - 1u;
                for (uint32_t c = (uint32_t)lane; c < ncand; c += kWave) {
                    const uint32_t kc = s.cand[c];
                    if ((kc & himask) == prefix) atomicAdd(&s.hl[l][(kc >> nshift) & dmask], 1u);
                }
                find_digit_p<4>(s.hl[l], kr, lane, dg, kr, cnt);
                prefix |= dg << nshift;
                himask |= dmask << nshift;
                shift = nshift;
                ++l;
            }
            if (lane == 0) { s.res[0] = prefix; s.res[1] = kr; s.res[2] = cnt; }
        }
        __syncthreads();
        prefix = s.res[0]; kr = s.res[1]; cnt = s.res[2];
      }
    } else {
        // One digit left, or many keys (ties, zeros): all wavefronts count
        // each digit and search its 256 bins.
        int shift = S1, l = 0;
        while (shift > 0) {
            const int nshift = shift > 8 ? shift - 8 : 0;
            const uint32_t dmask = (1u << (shift - nshift)) - 1u;
            count_level(s.hl[l], prefix, himask, nshift, dmask);
            __syncthreads();
            find_digit_p<4>(s.hl[l], kr, lane, dg, kr, cnt);
            prefix |= dg << nshift;
            himask |= dmask << nshift;
            shift = nshift;
            ++l;
        }
    }
    tau = prefix;
    kr_out = kr;
    eqtot = cnt;   // the last bin holds exactly the keys equal to tau
}

}  // namespace sel
}  // namespace qs
