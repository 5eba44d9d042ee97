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

// A workgroup barrier that orders LDS accesses only: global loads in flight
// stay in flight (__syncthreads() waits for them to land first).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// No-op level-1 hook of select_desc31 and select15_masks.
struct NoLevel1Hook {
    template <typename... A>
    __device__ __forceinline__ void operator()(A...) const {}
};

// Exclusive prefix over the threads of a workgroup (in thread order) of one
// count per thread; `tot` receives the total.  Two barriers (with LDS_ONLY,
// barriers that order LDS only: the caller's global loads stay in flight).
template <int NT, bool LDS_ONLY = false>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, int tid,
                                                    uint32_t& tot) {
    constexpr int NW = NT / sel::kWave;
    const int lane = tid & (sel::kWave - 1), wave = tid / sel::kWave;
    const uint32_t inc = sel::wave_incl_scan_dpp(v);
    if (lane == sel::kWave - 1) wsum[wave] = inc;
    if constexpr (LDS_ONLY) lds_barrier(); else __syncthreads();
    uint32_t before = 0, t = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t c = wsum[w];
        before += w < wave ? c : 0u;
        t += c;
    }
    if constexpr (LDS_ONLY) lds_barrier(); else __syncthreads();   // wsum may be reused after this
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
// Three or four barriers, no broadcast of the result; they order LDS only, so
// global loads the caller has in flight stay in flight.  The hook is called
// (uniformly) with each row's level-1 boundary bin: every key whose 8 high
// bits exceed it is selected, whatever level 2 finds.  L must be zeroed, and
// a barrier passed, before the call.
constexpr int kH1Pitch = 256 + 16;

template <int BT, int NW>
struct Sel15Lds {
    uint32_t h1[BT][4][kH1Pitch];   // four copies (by lane % 4): the few exponent bins
                                    // of an activation would serialise one copy's
                                    // atomics; the pitch puts a bin's copies on
                                    // different banks
    uint32_t h2[BT][128];
    uint32_t tie[BT][NW];
};

template <int NT, int BT, int E, typename Hook = NoLevel1Hook>
__device__ __forceinline__ void select15_masks(const uint32_t (&key)[BT][E], int ntok, int64_t k,
                                               Sel15Lds<BT, NT / 64>& L, int tid,
                                               uint32_t (&selm)[BT], Hook level1 = Hook()) {
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
    lds_barrier();
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
        level1(t, b1[t]);   // keys of level-1 bins above b1 are selected for sure
#pragma unroll
        for (int e2 = 0; e2 < E; ++e2)
            if (key[t][e2] != sel::kInvalid && (key[t][e2] >> 7) == b1[t])
                atomicAdd(&L.h2[t][key[t][e2] & 127u], 1u);
    }
    lds_barrier();
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
    if (ties) lds_barrier();   // uniform
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

// ---------------------------------------------------------------------------
// Descriptor (tau, cutoff) of the top-k of one row of 31-bit keys (fp32
// magnitudes) held by a workgroup, for kernels that select a row that a
// previous launch wrote (the FFN intermediate h; Turbo Sparse summary, Eq. 3-4:
// the top-k% of h by |h| before W_down).  Every wavefront scans each
// histogram itself, so no wavefront waits for another's search:
//   level 1: bits 30..20 of the nonzero keys (2048 bins: an exponent and three
//            mantissa bits, so an activation's few exponents spread out); zero
//            keys are not counted, so a row that is half zeros adds no
//            conflicting atomics on one bin;
//   level 2: bits 19..10 of the keys in level 1's boundary bin, which the same
//            pass also copies, with their indices, into a short list;
//   finish:  the few listed keys that share level 2's boundary bin are ranked
//            against each other inside each wavefront (key descending, then
//            index ascending): the k-th is tau and its index + 1 the cutoff;
//   else:    (a long list, many equal keys) level 3 on bits 9..0, and where
//            some keys equal to tau stay out, a block prefix count of them in
//            index order.
// A boundary bin that is taken whole ends the search early: tau is then one
// below the bin's smallest key and the cutoff 0.  Two barriers in the usual
// case, besides the one after the caller clears the histograms; they order
// LDS only, so global loads the caller has in flight stay in flight.  The
// hook is called (uniformly) with level 1's boundary bin: every key whose
// bits 30..20 exceed it is selected, whatever the later levels find.
// ---------------------------------------------------------------------------
constexpr int kS31Cap = 256;   // listed keys of level 1's boundary bin

template <int NQ, int NW>
struct Sel31Lds {
    uint32_t h1[2048];
    uint32_t h2[1024];
    uint32_t h3[1024];
    uint32_t nc;               // listed keys
    uint32_t cut;              // the tie search's result
    uint32_t pad[2];
    uint32_t ckey[kS31Cap], cidx[kS31Cap];
    uint32_t wkey[NW][64], widx[NW][64];   // each wavefront's finishing candidates
    uint32_t tie[NQ][NW];
};

// Clear what select_desc31 expects zeroed (h1 .. nc); a barrier must follow.
template <int NT, int NQ>
__device__ __forceinline__ void sel31_clear(Sel31Lds<NQ, NT / 64>& L, int tid) {
    constexpr int N4 = (2048 + 1024 + 1024 + 4) / 4;
    uint4* p = reinterpret_cast<uint4*>(&L.h1[0]);
    for (int i = tid; i < N4; i += NT) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Descending search of a histogram of 256 NC bins.  False (uniform) when
// fewer than kr keys are counted; else the bin that holds the kr-th largest
// counted key, the rank of that key inside its bin (1-based) and the bin's
// count.  Every read is a 16-byte load with the lanes on consecutive 16-byte
// blocks (a lane owning a long run of bins would put all lanes of a load on
// the same banks): the chunk totals first, then the chunk that holds the
// key, where lane l owns bins 255 - 4 l - i (i = 0 .. 3).
template <int NC>
__device__ __forceinline__ bool desc_bin(const uint32_t* h, uint32_t kr, int lane, uint32_t& digit,
                                         uint32_t& rank, uint32_t& cnt, uint32_t& total) {
    uint32_t t[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const uint4 v = *reinterpret_cast<const uint4*>(&h[256 * c + 4 * lane]);
        t[c] = (uint32_t)__builtin_amdgcn_readlane((int)sel::wave_incl_scan_dpp(v.x + v.y + v.z + v.w), 63);
    }
    total = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) total += t[c];
    if (kr > total) return false;
    int cs = 0;
    uint32_t above = 0;
#pragma unroll
    for (int c = NC - 1; c >= 0; --c) {   // uniform
        if (kr <= above + t[c]) { cs = c; break; }
        above += t[c];
    }
    const uint32_t kc = kr - above;
    const uint4 v = *reinterpret_cast<const uint4*>(&h[256 * cs + 252 - 4 * lane]);
    const uint32_t c4[4] = {v.w, v.z, v.y, v.x};   // descending bins
    const uint32_t lsum = c4[0] + c4[1] + c4[2] + c4[3];
    const uint32_t incl = sel::wave_incl_scan_dpp(lsum);
    const uint32_t excl = incl - lsum;
    const int src = (int)__builtin_ctzll(__ballot(excl < kc && kc <= incl));
    uint32_t e = excl, dg = 0, rk = 0, cn = 0;
    bool found = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (!found && e < kc && kc <= e + c4[i]) {
            found = true;
            dg = (uint32_t)(256 * cs + 255 - 4 * lane - i);
            rk = kc - e;
            cn = c4[i];
        }
        e += c4[i];
    }
    digit = (uint32_t)__builtin_amdgcn_readlane((int)dg, src);
    rank = (uint32_t)__builtin_amdgcn_readlane((int)rk, src);
    cnt = (uint32_t)__builtin_amdgcn_readlane((int)cn, src);
    return true;
}

// Thread t holds key[4 q + e] = the key of entry q * 4 NT + 4 t + e, and 0
// past the row end of n entries (zero keys are never counted, and as ties
// they come after every entry of the row).  L cleared by sel31_clear, then a
// barrier.
// Returns, uniform over the workgroup: entry j is among the top k iff key_j >
// tau, or key_j == tau and j < cutoff.
template <int NT, int NQ, typename Hook = NoLevel1Hook>
__device__ __forceinline__ void select_desc31(const uint32_t (&key)[4 * NQ], int64_t n, int64_t k,
                                              Sel31Lds<NQ, NT / 64>& L, int tid, uint32_t& tau_out,
                                              uint32_t& cut_out, Hook level1 = Hook()) {
    constexpr int NW = NT / 64, KPT = 4 * NQ;
    constexpr uint32_t kAll = 0x7FFFFFFFu;
    const int lane = tid & 63, wave = tid / 64;
    if (k <= 0) { tau_out = kAll; cut_out = 0; return; }   // nothing (keys are < 2^31 - 1 or NaN)
    if (k >= n) { tau_out = 0; cut_out = kAll; return; }   // everything

#pragma unroll
    for (int i = 0; i < KPT; ++i)
        if (key[i] != 0u) atomicAdd(&L.h1[key[i] >> 20], 1u);
    lds_barrier();

    uint32_t tau = 0, need = 0, eqn = 0;
    uint32_t b1, r1, c1, tot;
    const bool found1 = desc_bin<8>(L.h1, (uint32_t)k, lane, b1, r1, c1, tot);
    if (found1) level1(b1);   // keys of level-1 bins above b1 are selected for sure
    if (!found1) {
        // Fewer than k nonzero keys: all of them, and the first zeros.
        tau = 0; need = (uint32_t)k - tot; eqn = (uint32_t)n - tot;
    } else if (r1 == c1) {
        // The boundary bin is taken whole: every key >= its lowest (a key
        // counted in bin 0 is nonzero).
        tau_out = b1 == 0 ? 0u : (b1 << 20) - 1u; cut_out = 0; return;
    } else {
        // Level 2, and the list of level 1's boundary keys (each listed with
        // one LDS atomic: they are few).  A zero key matches no boundary bin:
        // key >= lo1 (lo1 = 1 only for bin 0) excludes it, a test the
        // compiler cannot merge with level 1's, whose lane masks would
        // otherwise stay alive, one per key, across the search.
        const bool list = c1 <= (uint32_t)kS31Cap;   // uniform
        const uint32_t lo1 = b1 == 0 ? 1u : 0u;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            if ((key[i] >> 20) == b1 && key[i] >= lo1) {
                atomicAdd(&L.h2[(key[i] >> 10) & 1023u], 1u);
                if (list) {
                    const uint32_t pos = atomicAdd(&L.nc, 1u);
                    L.ckey[pos] = key[i];
                    L.cidx[pos] = (uint32_t)((i / 4) * 4 * NT + 4 * tid + (i % 4));
                }
            }
        }
        lds_barrier();
        uint32_t b2, r2, c2;
        desc_bin<4>(L.h2, r1, lane, b2, r2, c2, tot);   // r1 <= c1 = the level's total
        const uint32_t pre2 = (b1 << 10) | b2;            // the top 21 key bits
        if (r2 == c2) {
            const uint32_t lo = pre2 << 10;
            tau_out = lo == 0 ? 0u : lo - 1u; cut_out = 0; return;
        }
        if (list && c2 <= 64u) {
            // The c2 keys of the boundary bin, gathered from the list into
            // this wavefront's slots (lane i takes the i-th), then ranked.
            uint32_t base = 0;
            for (uint32_t ch = 0; ch < c1; ch += 64) {   // uniform
                const uint32_t e = ch + (uint32_t)lane;
                const uint32_t kv = e < c1 ? L.ckey[e] : sel::kInvalid;
                const bool m = e < c1 && (kv >> 10) == pre2;
                const uint64_t bm = __ballot(m);
                if (m) {
                    const uint32_t slot = base + sel::popc_below(bm);
                    L.wkey[wave][slot] = kv;
                    L.widx[wave][slot] = L.cidx[e];
                }
                base += (uint32_t)__popcll(bm);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const bool have = lane < (int)c2;
            const uint32_t ck = have ? L.wkey[wave][lane] : 0u;
            const uint32_t cj = have ? L.widx[wave][lane] : 0u;
            uint32_t rank = 0;
            for (uint32_t m = 0; m < c2; ++m) {   // uniform trip count
                const uint32_t km = (uint32_t)__builtin_amdgcn_readlane((int)ck, (int)m);
                const uint32_t jm = (uint32_t)__builtin_amdgcn_readlane((int)cj, (int)m);
                rank += (km > ck || (km == ck && jm < cj)) ? 1u : 0u;
            }
            const int src = (int)__builtin_ctzll(__ballot(have && rank == r2 - 1u));
            tau_out = (uint32_t)__builtin_amdgcn_readlane((int)ck, src);
            cut_out = (uint32_t)__builtin_amdgcn_readlane((int)cj, src) + 1u;
            return;
        }
        // Level 3: the low ten bits.
        const uint32_t lo2 = pre2 == 0 ? 1u : 0u;
#pragma unroll
        for (int i = 0; i < KPT; ++i)
            if ((key[i] >> 10) == pre2 && key[i] >= lo2) atomicAdd(&L.h3[key[i] & 1023u], 1u);
        lds_barrier();
        uint32_t b3;
        desc_bin<4>(L.h3, r2, lane, b3, need, eqn, tot);
        tau = (pre2 << 10) | b3;
        if (need == eqn) { tau_out = tau; cut_out = kAll; return; }
    }

    // Some keys equal to tau stay out: the need-th of them in index order
    // (runs in (q, thread, e) order) ends the selection.  The ties are kept
    // as bits, 4 per run, so the keys are tested once.
    uint32_t tb[NQ], incl[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        tb[q] = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) tb[q] |= (key[4 * q + e] == tau ? 1u : 0u) << e;
        incl[q] = sel::wave_incl_scan_dpp((uint32_t)__popc(tb[q]));
        if (lane == 63) L.tie[q][wave] = incl[q];
    }
    lds_barrier();
    uint32_t base = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        uint32_t before = 0, qt = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint32_t t = L.tie[q][w];
            before += w < wave ? t : 0u;
            qt += t;
        }
        const uint32_t c = (uint32_t)__popc(tb[q]);
        const uint32_t r = base + before + incl[q] - c;   // ties before this run
        if (r < need && need <= r + c) {
            uint32_t bits = tb[q];
            for (uint32_t s2 = r + 1; s2 < need; ++s2) bits &= bits - 1u;   // drop the lower ties
            L.cut = (uint32_t)(q * 4 * NT + 4 * tid + __builtin_ctz(bits)) + 1u;
        }
        base += qt;
    }
    lds_barrier();
    tau_out = tau;
    cut_out = L.cut;
}

__device__ __forceinline__ bool selected(uint32_t key, uint32_t j, uint32_t tau, uint32_t cutoff) {
    return key > tau || (key == tau && j < cutoff);
}

}  // namespace rowsel
}  // namespace qs
