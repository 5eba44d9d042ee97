// Per-row top-K selection by |x| with ties to the lower index (gfx950).
//
// Q-Sparse news article (zxwl-tech.com), section "Sparsification with the
// Top-K function": take |X|, find the K entries of largest magnitude, build
// a mask of X's shape that is 1 there, and use X (.) M in place of X.  Ties
// (not covered by the pages) go to the lower index.
//
// One workgroup per row.  The row's raw words are staged in LDS, then an
// MSD radix select on the magnitude key (8-bit digits, per-wave-group LDS
// histograms, a descending block scan over the 256 bins) finds tau, the key
// of the K-th largest entry, and how many entries equal to tau are taken.
// A final pass walks the row in index order in chunks of one workgroup: two
// wavefront ballots (key > tau, key == tau) and mbcnt prefix counts give
// each tie its rank and each selected entry its slot in the ascending index
// list, with one barrier per chunk (double-buffered wave totals).
//
// The quantised variant (KEY_Q8) first quantises the fp32 row to int8
// (absmax, IEEE binary32 with round-to-nearest-even at every step; Q-Sparse
// news article, Top-K section: activations are quantised before top-K with
// an epsilon-guarded denominator) and then selects on |q|.
#include "qs_internal.h"
#include "qs_select.h"
#include "qs_rowsel.h"

namespace qs {
namespace {

constexpr int kWave = 64;

// Side jobs of the selection launch, done before anything else: workgroup 0
// clears the split-K counters of the gather that follows, and the workgroup
// of row r clears row r of the buffers that the next kernel adds into.
template <int NT>
__device__ __forceinline__ void clear_side_buffers(const TopkArgs& a, int r, int tid) {
    if (r == 0 && a.zero_ptr != nullptr)
        for (int i = tid; i < a.n_zero; i += NT) a.zero_ptr[i] = 0;
    int32_t* const zr[2] = {a.zero_rows, a.zero_rows2};
#pragma unroll
    for (int b = 0; b < 2; ++b)
        if (zr[b] != nullptr)
            for (int64_t i = tid; i < a.zero_row_len / 4; i += NT)
                reinterpret_cast<uint4*>(zr[b] + (int64_t)r * a.zero_row_len)[i] = make_uint4(0u, 0u, 0u, 0u);
}
constexpr int kNSub = 4;               // LDS sub-histograms (spread atomic contention)
constexpr int64_t kStageMaxD = 14336;  // raw words staged in LDS up to this row length

using sel::popc_below;
using sel::wave_incl_scan_dpp;
using sel::find_digit_p;
using sel::find_top_lane;

// Raw 32-bit word of element i, and its magnitude key.
template <int KK> struct Elem;

template <> struct Elem<KEY_F32> {
    static constexpr int kKeyBits = 31;
    __device__ static uint32_t load(const void* x, int64_t i, float) {
        return reinterpret_cast<const uint32_t*>(x)[i];
    }
    __device__ static uint32_t key(uint32_t raw) { return raw & 0x7FFFFFFFu; }
};

template <> struct Elem<KEY_BF16> {
    static constexpr int kKeyBits = 15;
    __device__ static uint32_t load(const void* x, int64_t i, float) {
        return reinterpret_cast<const uint16_t*>(x)[i];
    }
    __device__ static uint32_t key(uint32_t raw) { return raw & 0x7FFFu; }
};

template <> struct Elem<KEY_I8> {
    static constexpr int kKeyBits = 8;
    __device__ static uint32_t load(const void* x, int64_t i, float) {
        return (uint32_t)(int32_t)reinterpret_cast<const int8_t*>(x)[i];
    }
    __device__ static uint32_t key(uint32_t raw) {
        int32_t v = (int32_t)raw;
        return (uint32_t)(v < 0 ? -v : v);
    }
};

template <> struct Elem<KEY_Q8> {
    static constexpr int kKeyBits = 8;
    // q = clamp(rint(fl32(x * s)), -128, 127)
    __device__ static uint32_t load(const void* x, int64_t i, float s) {
        float v = reinterpret_cast<const float*>(x)[i];
        float r = rintf(__fmul_rn(v, s));
        r = fminf(fmaxf(r, -128.0f), 127.0f);
        return (uint32_t)(int32_t)r;
    }
    __device__ static uint32_t key(uint32_t raw) { return Elem<KEY_I8>::key(raw); }
};

// Raw words of a whole row through one buffer resource: all loads are issued
// back to back (no per-entry branch), and entries past the row end read 0.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <int KK>
__device__ __forceinline__ uint32_t buffer_raw(__amdgpu_buffer_rsrc_t rs, uint32_t j) {
    if constexpr (KK == KEY_BF16)
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, j * 2u, 0, 0);
    else if constexpr (KK == KEY_I8)
        return (uint32_t)(int32_t)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(rs, j, 0, 0);
    else
        return __builtin_amdgcn_raw_buffer_load_b32(rs, j * 4u, 0, 0);
}
template <int KK> constexpr int elem_bytes() {
    return KK == KEY_BF16 ? 2 : (KK == KEY_I8 ? 1 : 4);
}

template <int KK, int XK>
__device__ __forceinline__ void store_xs(void* xs, int64_t i, uint32_t raw, bool sel) {
    if constexpr (XK == XS_F32) {
        float v = 0.0f;
        if (sel) {
            if constexpr (KK == KEY_F32) v = __uint_as_float(raw);
            else if constexpr (KK == KEY_BF16) v = __uint_as_float(raw << 16);
            else v = (float)(int32_t)raw;
        }
        reinterpret_cast<float*>(xs)[i] = v;
    } else if constexpr (XK == XS_BF16) {
        reinterpret_cast<uint16_t*>(xs)[i] = sel ? (uint16_t)raw : (uint16_t)0;
    } else if constexpr (XK == XS_I8) {
        reinterpret_cast<int8_t*>(xs)[i] = sel ? (int8_t)(int32_t)raw : (int8_t)0;
    }
}

template <int NT, int KK, int XK, bool STAGED>
__global__ __launch_bounds__(NT) void topk_rows_kernel(TopkArgs a) {
    constexpr int NW = NT / kWave;
    extern __shared__ uint32_t s_raw[];                 // [d] when STAGED
    __shared__ uint32_t s_hist[kNSub][256];
    __shared__ uint32_t s_scan[4];
    __shared__ uint32_t s_gt[2][NW], s_eq[2][NW];
    __shared__ uint32_t s_digit, s_kr;
    __shared__ float s_max[NW];

    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int64_t d = a.d;
    const int64_t k = a.k;
    const int64_t row0 = (int64_t)r * d;

    clear_side_buffers<NT>(a, r, tid);

    // Quantisation scale (KEY_Q8): gamma = max|x| (exact), s = 127 / (gamma + eps).
    float scale = 0.0f;
    if constexpr (KK == KEY_Q8) {
        const float* xr = reinterpret_cast<const float*>(a.x) + row0;
        float m = 0.0f;
        for (int64_t j = tid; j < d; j += NT) m = fmaxf(m, fabsf(xr[j]));
        for (int off = kWave / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        if (lane == 0) s_max[wave] = m;
        __syncthreads();
        float g = s_max[0];
        for (int w = 1; w < NW; ++w) g = fmaxf(g, s_max[w]);
        scale = __fdiv_rn(127.0f, __fadd_rn(g, 1e-5f));
        if (tid == 0 && a.xscale != nullptr) a.xscale[r] = scale;
    }

    if constexpr (STAGED) {
        for (int64_t j = tid; j < d; j += NT) {
            uint32_t raw = Elem<KK>::load(a.x, row0 + j, scale);
            s_raw[j] = raw;
            if constexpr (KK == KEY_Q8)
                if (a.xq != nullptr) a.xq[row0 + j] = (int8_t)(int32_t)raw;
        }
        __syncthreads();
    } else {
        if constexpr (KK == KEY_Q8)
            if (a.xq != nullptr)
                for (int64_t j = tid; j < d; j += NT)
                    a.xq[row0 + j] = (int8_t)(int32_t)Elem<KK>::load(a.x, row0 + j, scale);
    }
    auto raw_at = [&](int64_t j) -> uint32_t {
        if constexpr (STAGED) return s_raw[j];
        else return Elem<KK>::load(a.x, row0 + j, scale);
    };

    // ---- MSD radix select: tau and the number kr of tau-ties to take.
    uint32_t prefix = 0, himask = 0, kr = (uint32_t)k;
    if (k > 0) {
        constexpr int kPasses = (Elem<KK>::kKeyBits + 7) / 8;
#pragma unroll 1
        for (int p = kPasses - 1; p >= 0; --p) {
            const int shift = 8 * p;
            for (int i = tid; i < kNSub * 256; i += NT) (&s_hist[0][0])[i] = 0;
            __syncthreads();
            uint32_t* hsub = s_hist[wave % kNSub];
            for (int64_t j = tid; j < d; j += NT) {
                uint32_t key = Elem<KK>::key(raw_at(j));
                if ((key & himask) == prefix) atomicAdd(&hsub[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            // Threads 0..255 own bins in descending order; inclusive scan gives
            // the number of candidates with digit >= bin.
            uint32_t v = 0, incl = 0;
            if (tid < 256) {
                const int b = 255 - tid;
#pragma unroll
                for (int q = 0; q < kNSub; ++q) v += s_hist[q][b];
                incl = v;
#pragma unroll
                for (int off = 1; off < kWave; off <<= 1) {
                    uint32_t n = __shfl_up(incl, off);
                    if (lane >= off) incl += n;
                }
                if (lane == kWave - 1) s_scan[wave] = incl;
            }
            __syncthreads();
            if (tid < 256) {
                uint32_t base = 0;
                for (int w = 0; w < wave; ++w) base += s_scan[w];
                incl += base;
                const uint32_t excl = incl - v;
                if (excl < kr && kr <= incl) {
                    s_digit = (uint32_t)(255 - tid);
                    s_kr = kr - excl;
                }
            }
            __syncthreads();
            prefix |= s_digit << shift;
            himask |= 0xFFu << shift;
            kr = s_kr;
        }
    }
    const uint32_t tau = (k > 0) ? prefix : 0xFFFFFFFFu;

    // ---- Ordered pass: tie ranks, selection, compaction, outputs.
    uint32_t eq_run = 0, sel_run = 0;
    int buf = 0;
    for (int64_t base = 0; base < d; base += NT) {
        const int64_t j = base + tid;
        const bool valid = j < d;
        const uint32_t raw = valid ? raw_at(j) : 0u;
        const uint32_t key = Elem<KK>::key(raw);
        const bool gt = valid && k > 0 && key > tau;
        const bool eq = valid && k > 0 && key == tau;
        const uint64_t bgt = __ballot(gt);
        const uint64_t beq = __ballot(eq);
        if (lane == 0) {
            s_gt[buf][wave] = (uint32_t)__popcll(bgt);
            s_eq[buf][wave] = (uint32_t)__popcll(beq);
        }
        __syncthreads();
        uint32_t eq_before = eq_run, sel_before = sel_run;
        uint32_t my_eq = 0, my_sel = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint32_t g = s_gt[buf][w], e = s_eq[buf][w];
            const uint32_t take = kr > eq_before ? min(e, kr - eq_before) : 0u;
            if (w == wave) { my_eq = eq_before; my_sel = sel_before; }
            eq_before += e;
            sel_before += g + take;
        }
        const uint32_t eq_rank = my_eq + popc_below(beq);
        const bool sel = gt || (eq && eq_rank < kr);
        const uint64_t bsel = __ballot(sel);
        if (valid) {
            const uint32_t pos = my_sel + popc_below(bsel);
            if (a.mask != nullptr) a.mask[row0 + j] = sel ? 1 : 0;
            if constexpr (XK != XS_NONE)
                if (a.xs != nullptr) store_xs<KK, XK>(a.xs, row0 + j, raw, sel);
            if (sel && pos < (uint32_t)k && a.idx != nullptr) a.idx[(int64_t)r * a.idx_stride + pos] = (int32_t)j;
            if (eq && eq_rank + 1 == kr && a.cutoff != nullptr) a.cutoff[r] = (int32_t)(j + 1);
        }
        eq_run = eq_before;
        sel_run = sel_before;
        buf ^= 1;
    }
    if (tid == 0) {
        if (a.tau != nullptr) a.tau[r] = tau;
        if (k == 0 && a.cutoff != nullptr) a.cutoff[r] = 0;
        if (a.count != nullptr) a.count[r] = (int32_t)k;
    }
}

// ---------------------------------------------------------------------------
// Register-resident variant for rows of up to EPT * NT entries (the common
// case), NT = 256.  Thread t keeps entries t, t + NT, ... in registers.  The
// threshold key is found bit by bit from the most significant key bit: for
// each bit, one compare per entry, a wavefront ballot and a scalar popcount
// count the candidates that keep the current prefix with that bit set; the
// four per-wave counts meet in LDS behind one barrier (double-buffered by bit
// parity).  No atomics, so skewed key distributions (many equal exponents)
// cost nothing extra.  The ordered output pass needs three barriers in all:
// per-(chunk, wave) counts of keys above and equal to tau go to LDS, wave 0
// turns them into exclusive prefixes (tie ranks and output slots) with two
// wavefront scans, and every thread then places its entries.  Entries past
// the row end carry bit 31, which no valid key has, so they never match a
// prefix or tie with tau.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, int lane) {
    uint32_t incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t n = __shfl_up(incl, off);
        if (lane >= off) incl += n;
    }
    return incl - v;
}

template <int NT, int EPT, int KK, int XK>
__global__ __launch_bounds__(NT) void topk_reg_kernel(TopkArgs a) {
    constexpr int NW = NT / kWave;
    constexpr int NE = EPT * NW;                  // (chunk, wave) entries
    constexpr int PER = (NE + kWave - 1) / kWave; // entries per lane in the scan
    constexpr uint32_t kInvalid = 0x80000000u;
    constexpr int kCap = 1024;                    // compacted candidates
    __shared__ uint32_t s_cnt[2][NW];
    __shared__ uint32_t s_g[NE], s_e[NE], s_gb[NE], s_eb[NE];
    __shared__ uint32_t s_cand[kCap];
    __shared__ uint32_t s_ncand, s_res[2];
    __shared__ float s_max[NW];

    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int64_t d = a.d;
    const int64_t k = a.k;
    const int64_t row0 = (int64_t)r * d;
    const int nch = (int)((d + NT - 1) / NT);     // chunks holding entries (<= EPT)

    clear_side_buffers<NT>(a, r, tid);

    // Load the row: every load issued before any is used.
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(a.x)) + row0 * elem_bytes<KK>(), (short)0,
        (int)(d * elem_bytes<KK>()), 0x00020000);
    uint32_t raw[EPT], key[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) raw[i] = buffer_raw<KK>(rs, (uint32_t)(i * NT + tid));

    float scale = 0.0f;
    if constexpr (KK == KEY_Q8) {
        // gamma = max |x| (exact), s = 127 / (gamma + eps), q = rint(x s)
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < EPT; ++i) m = fmaxf(m, fabsf(__uint_as_float(raw[i])));
        for (int off = kWave / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        if (lane == 0) s_max[wave] = m;
        __syncthreads();
        float g = s_max[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) g = fmaxf(g, s_max[w]);
        scale = __fdiv_rn(127.0f, __fadd_rn(g, 1e-5f));
        if (tid == 0 && a.xscale != nullptr) a.xscale[r] = scale;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            float q = rintf(__fmul_rn(__uint_as_float(raw[i]), scale));
            q = fminf(fmaxf(q, -128.0f), 127.0f);
            raw[i] = (uint32_t)(int32_t)q;
            const int64_t j = (int64_t)i * NT + tid;
            if (a.xq != nullptr && j < d) a.xq[row0 + j] = (int8_t)(int32_t)q;
        }
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i)
        key[i] = (int64_t)i * NT + tid < d ? Elem<KK>::key(raw[i]) : kInvalid;

    // ---- bitwise MSD select: tau and the number kr of tau-ties to take.
    // The top kFull key bits are resolved over the whole row; the entries
    // still matching the prefix (typically ~1% of the row) are then compacted
    // into LDS and wave 0 resolves the remaining bits alone, without barriers.
    // If more than kCap entries survive, the whole block keeps going instead.
    constexpr int KB = Elem<KK>::kKeyBits;
    constexpr int kFull = KB > 12 ? (KB > 16 ? 12 : 10) : KB;
    uint32_t prefix = 0, himask = kInvalid, kr = (uint32_t)k;
    auto full_pass = [&](int b) {
        const uint32_t bit = 1u << b;
        const uint32_t mb = himask | bit, cb = prefix | bit;
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < EPT; ++i) c += (uint32_t)__popcll(__ballot((key[i] & mb) == cb));
        // readfirstlane is convergent: it keeps the popcounts out of the
        // lane-0 branch (otherwise every ballot mask stays live in SGPRs).
        c = __builtin_amdgcn_readfirstlane(c);
        const int par = b & 1;
        if (lane == 0) s_cnt[par][wave] = c;
        __syncthreads();
        uint32_t total = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) total += s_cnt[par][w];
        if (total >= kr) prefix = cb;
        else kr -= total;
        himask |= bit;
    };
    if (k > 0) {
        int b = KB - 1;
#pragma unroll 1
        for (; b >= KB - kFull; --b) full_pass(b);
        if (b >= 0) {
            if (tid == 0) s_ncand = 0;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < EPT; ++i) {
                const bool m = (key[i] & himask) == prefix;
                const uint64_t bm = __ballot(m);
                const uint32_t n = (uint32_t)__popcll(bm);
                uint32_t base = 0;
                if (lane == 0 && n != 0) base = atomicAdd(&s_ncand, n);
                base = __shfl(base, 0);
                const uint32_t pos = base + popc_below(bm);
                if (m && pos < (uint32_t)kCap) s_cand[pos] = key[i];
            }
            __syncthreads();
            const uint32_t nc = s_ncand;
            if (nc <= (uint32_t)kCap) {
                if (wave == 0) {
                    uint32_t ck[kCap / kWave];
#pragma unroll
                    for (int q = 0; q < kCap / kWave; ++q) {
                        const uint32_t n = (uint32_t)(q * kWave + lane);
                        ck[q] = n < nc ? s_cand[n] : kInvalid;
                    }
#pragma unroll 1
                    for (; b >= 0; --b) {
                        const uint32_t bit = 1u << b;
                        const uint32_t mb = himask | bit, cb = prefix | bit;
                        uint32_t c = 0;
#pragma unroll
                        for (int q = 0; q < kCap / kWave; ++q)
                            c += (uint32_t)__popcll(__ballot((ck[q] & mb) == cb));
                        if (c >= kr) prefix = cb;
                        else kr -= c;
                        himask |= bit;
                    }
                    if (lane == 0) { s_res[0] = prefix; s_res[1] = kr; }
                }
                __syncthreads();
                prefix = s_res[0];
                kr = s_res[1];
            } else {
#pragma unroll 1
                for (; b >= 0; --b) full_pass(b);
            }
        }
    }
    const uint32_t tau = (k > 0) ? prefix : 0xFFFFFFFFu;

    // ---- ordered output.  Phase 1: per-(chunk, wave) counts.
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        if (i < nch) {
            const bool gt = k > 0 && key[i] != kInvalid && key[i] > tau;
            const bool eq = k > 0 && key[i] == tau;
            const uint32_t g = (uint32_t)__popcll(__ballot(gt));
            const uint32_t e = (uint32_t)__popcll(__ballot(eq));
            if (lane == 0) { s_g[i * NW + wave] = g; s_e[i * NW + wave] = e; }
        }
    }
    __syncthreads();
    // Phase 2: wave 0 scans the entries in (chunk, wave) order.  Ties are
    // taken in index order until kr of them are in; an entry's selected
    // count is its keys above tau plus the ties it contributes.
    if (wave == 0) {
        const int ne = nch * NW;
        uint32_t e_loc[PER], g_loc[PER], esum = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int n = lane * PER + q;
            e_loc[q] = n < ne ? s_e[n] : 0u;
            g_loc[q] = n < ne ? s_g[n] : 0u;
            esum += e_loc[q];
        }
        uint32_t eb = wave_excl_scan(esum, lane);
        uint32_t sel_loc[PER], ssum = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const uint32_t take = kr > eb ? min(e_loc[q], kr - eb) : 0u;
            const int n = lane * PER + q;
            if (n < ne) s_eb[n] = eb;
            eb += e_loc[q];
            sel_loc[q] = g_loc[q] + take;
            ssum += sel_loc[q];
        }
        uint32_t sb = wave_excl_scan(ssum, lane);
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int n = lane * PER + q;
            if (n < ne) s_gb[n] = sb;
            sb += sel_loc[q];
        }
    }
    __syncthreads();
    // Phase 3: place the entries.  The prefixes are read for every chunk up
    // front (entries past nch are never used), so no LDS round trip sits on
    // the per-chunk dependency chain.
    uint32_t ebv[EPT], gbv[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        ebv[i] = s_eb[i * NW + wave];
        gbv[i] = s_gb[i * NW + wave];
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        if (i < nch) {
            const int64_t j = (int64_t)i * NT + tid;
            const bool valid = key[i] != kInvalid;
            const bool gt = k > 0 && valid && key[i] > tau;
            const bool eq = k > 0 && key[i] == tau;
            const uint64_t beq = __ballot(eq);
            const uint32_t eq_rank = ebv[i] + popc_below(beq);
            const bool sel = gt || (eq && eq_rank < kr);
            const uint64_t bsel = __ballot(sel);
            if (valid) {
                const uint32_t pos = gbv[i] + popc_below(bsel);
                if (a.mask != nullptr) a.mask[row0 + j] = sel ? 1 : 0;
                if constexpr (XK != XS_NONE)
                    if (a.xs != nullptr) store_xs<KK, XK>(a.xs, row0 + j, raw[i], sel);
                if (sel && pos < (uint32_t)k && a.idx != nullptr)
                    a.idx[(int64_t)r * a.idx_stride + pos] = (int32_t)j;
                if (eq && eq_rank + 1 == kr && a.cutoff != nullptr) a.cutoff[r] = (int32_t)(j + 1);
            }
        }
    }
    if (tid == 0) {
        if (a.tau != nullptr) a.tau[r] = tau;
        if (k == 0 && a.cutoff != nullptr) a.cutoff[r] = 0;
        if (a.count != nullptr) a.count[r] = (int32_t)k;
    }
}

// ---------------------------------------------------------------------------
// Vectorised variant (the main path): rows whose byte length is a multiple of
// 16 and that fit NQ runs per thread.  Thread t of 256 loads run q, the V
// entries [q * 256 V + t V, + V) of the row, with one 16-byte buffer load
// (V = 4 fp32, 8 bf16, 16 int8), so every load instruction of a wavefront
// reads 1 KiB contiguously.  Index order is (run, thread, entry).
//
// Select: 8-bit digits from the top of the key.  The first digit is counted
// over every entry (LDS histograms, one per wavefront, so that contention on
// frequent exponents stays inside a wave); a descending block scan of the 256
// bins finds the digit of the K-th largest key.  The entries that still
// match the prefix are compacted into LDS (per-wave ballot counts, one
// barrier, no atomics), and the remaining digits are counted over those
// candidates only.  Output: the tie ranks and output slots of all runs come
// from two block-wide scans over (run, thread) order (wave scans of every run
// at once, one barrier each), after which every thread writes its runs with
// vector stores.
// ---------------------------------------------------------------------------
// bf16 round-to-nearest-even of an fp32 value (finite inputs), as the
// 16-token MFMA gather's packing splits a coefficient into hi + lo.
__device__ __forceinline__ uint32_t frag_bf16_rne(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return b >> 16;
}

template <int KK> struct VecOf;
template <> struct VecOf<KEY_F32> { static constexpr int V = 4; };
template <> struct VecOf<KEY_Q8> { static constexpr int V = 4; };
template <> struct VecOf<KEY_BF16> { static constexpr int V = 8; };
template <> struct VecOf<KEY_I8> { static constexpr int V = 16; };

template <int KK>
__device__ __forceinline__ void unpack_raw(const u32x4_t& w, uint32_t* raw) {
    if constexpr (KK == KEY_F32 || KK == KEY_Q8) {
        raw[0] = w.x; raw[1] = w.y; raw[2] = w.z; raw[3] = w.w;
    } else if constexpr (KK == KEY_BF16) {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { raw[2 * i] = u[i] & 0xFFFFu; raw[2 * i + 1] = u[i] >> 16; }
    } else {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) raw[i] = (uint32_t)(int32_t)(int8_t)(u[i / 4] >> (8 * (i % 4)));
    }
}

// Every wavefront scans the whole 256-bin histogram (summed over the NW
// sub-histograms) from the top bin down and finds the bin that holds the
// kr-th largest key, so no second barrier is needed.  Lane l owns bins
// 255 - 4l - c (c = 0..3).  Returns the digit and the rank of the wanted key
// inside its bin.
template <int NS>
__device__ __forceinline__ void find_digit(const uint32_t (*h)[256], uint32_t kr, int lane,
                                           uint32_t& digit, uint32_t& kr_out) {
    uint32_t c4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int w = 0; w < NS; ++w) {
        const uint4 v = *reinterpret_cast<const uint4*>(&h[w][252 - 4 * lane]);   // bins 252+3-4l .. 252-4l
        c4[0] += v.w; c4[1] += v.z; c4[2] += v.y; c4[3] += v.x;                // descending order
    }
    const uint32_t lsum = c4[0] + c4[1] + c4[2] + c4[3];
    const uint32_t incl = wave_incl_scan_dpp(lsum);
    const uint32_t excl = incl - lsum;
    const bool mine = excl < kr && kr <= incl;
    const uint64_t bm = __ballot(mine);
    const int src = (int)__builtin_ctzll(bm);
    uint32_t e = excl, dg = 0, kk = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (dg == 0 && kk == 0 && e < kr && kr <= e + c4[c]) { dg = (uint32_t)(255 - 4 * lane - c); kk = kr - e; }
        e += c4[c];
    }
    digit = (uint32_t)__builtin_amdgcn_readlane((int)dg, src);
    kr_out = (uint32_t)__builtin_amdgcn_readlane((int)kk, src);
}

template <int NT, int NQ, int KK, int XK>
__global__ __launch_bounds__(NT) void topk_vec_kernel(TopkArgs a) {
    constexpr int NW = NT / kWave;
    constexpr int V = VecOf<KK>::V, CS = V * NT, EPT = NQ * V;
    constexpr int KB = Elem<KK>::kKeyBits;
    constexpr uint32_t kInvalid = sel::kInvalid;
    constexpr int ESZ = elem_bytes<KK>();
    __shared__ sel::SelectLds<KB> s_sel;
    __shared__ uint32_t s_tot[2][NQ][NW];
    __shared__ float s_max[NW];

    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int64_t d = a.d, k = a.k, row0 = (int64_t)r * d;

    sel::select_clear<NT, KB>(s_sel, tid);

    // ---- load runs (past the row end the buffer reads zero)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(a.x)) + row0 * ESZ, (short)0,
        (int)(d * ESZ), 0x00020000);
    uint32_t raw[EPT], key[EPT];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(
            rs, (uint32_t)((q * CS + V * tid) * ESZ), 0, 0);
        unpack_raw<KK>(w, raw + q * V);
    }
    auto run_valid = [&](int q) { return (int64_t)q * CS + V * tid < d; };   // d % V == 0
    // The side stores go out behind the row's loads, which start the critical chain.
    clear_side_buffers<NT>(a, r, tid);

    // Elementwise map of the row before the selection (the FFN intermediate
    // from raw projection sums): h = relu(u)^2, or relu(g)^2 * u with the
    // gate sums g in x2, in the same fp32 operations as the gather epilogue.
    if constexpr (KK == KEY_F32) {
        if (a.xform != XF_NONE) {
            uint32_t graw[EPT];
            if (a.xform == XF_RELU2_GLU) {
                const __amdgpu_buffer_rsrc_t rs2 = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<float*>(a.x2 + row0), (short)0, (int)(d * 4), 0x00020000);
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(
                        rs2, (uint32_t)((q * CS + V * tid) * 4), 0, 0);
                    unpack_raw<KK>(w, graw + q * V);
                }
            }
#pragma unroll
            for (int i = 0; i < EPT; ++i) {
                const float u = __uint_as_float(raw[i]);
                float hv;
                if (a.xform == XF_RELU2) {
                    hv = u > 0.0f ? __fmul_rn(u, u) : 0.0f;
                } else {
                    const float g = __uint_as_float(graw[i]);
                    hv = g > 0.0f ? __fmul_rn(__fmul_rn(g, g), u) : 0.0f;
                }
                raw[i] = __float_as_uint(hv);
            }
            if (a.h_out != nullptr) {
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    if (run_valid(q))
                        *reinterpret_cast<uint4*>(a.h_out + row0 + q * CS + V * tid) =
                            make_uint4(raw[q * V], raw[q * V + 1], raw[q * V + 2], raw[q * V + 3]);
            }
        }
    }

    if constexpr (KK == KEY_Q8) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < EPT; ++i) m = fmaxf(m, fabsf(__uint_as_float(raw[i])));
        for (int off = kWave / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        if (lane == 0) s_max[wave] = m;
        __syncthreads();
        float g = s_max[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) g = fmaxf(g, s_max[w]);
        const float scale = __fdiv_rn(127.0f, __fadd_rn(g, 1e-5f));
        if (tid == 0 && a.xscale != nullptr) a.xscale[r] = scale;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            uint32_t packed = 0;
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float qv = rintf(__fmul_rn(__uint_as_float(raw[q * V + e]), scale));
                qv = fminf(fmaxf(qv, -128.0f), 127.0f);
                raw[q * V + e] = (uint32_t)(int32_t)qv;
                packed |= ((uint32_t)(int32_t)qv & 0xFFu) << (8 * e);
            }
            if (a.xq != nullptr && run_valid(q))
                *reinterpret_cast<uint32_t*>(a.xq + row0 + q * CS + V * tid) = packed;
        }
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int e = 0; e < V; ++e)
            key[q * V + e] = run_valid(q) ? Elem<KK>::key(raw[q * V + e]) : kInvalid;
    __syncthreads();   // histograms cleared

    // ---- select
    uint32_t tau = 0xFFFFFFFFu, kr = (uint32_t)k, eqtot = 0;
    if (k > 0) sel::radix_select<NT, EPT, KB>(key, (uint32_t)k, s_sel, tid, tau, kr, eqtot);

    // ---- ordered output: two block scans over (run, thread) order.
    uint32_t eqc[NQ], gtc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        eqc[q] = 0; gtc[q] = 0;
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const uint32_t kk = key[q * V + e];
            eqc[q] += (k > 0 && kk == tau) ? 1u : 0u;
            gtc[q] += (k > 0 && kk != kInvalid && kk > tau) ? 1u : 0u;
        }
    }
    // exclusive prefix of cnt[] in (run, thread) order, into out[]
    auto block_scan = [&](const uint32_t* cnt, uint32_t* out, int buf) {
        uint32_t inc[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) inc[q] = wave_incl_scan_dpp(cnt[q]);
        if (lane == kWave - 1)
#pragma unroll
            for (int q = 0; q < NQ; ++q) s_tot[buf][q][wave] = inc[q];
        __syncthreads();
        uint32_t base = 0;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            uint32_t before = 0, tot = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const uint32_t t = s_tot[buf][q][w];
                before += w < wave ? t : 0u;
                tot += t;
            }
            out[q] = base + before + inc[q] - cnt[q];
            base += tot;
        }
    };
    // The tie ranks are needed only when some keys equal to tau stay out (or
    // the cutoff is asked for), the output slots only for the index list.
    uint32_t eqb[NQ], selc[NQ], selb[NQ];
    const bool all_ties = k > 0 && kr >= eqtot;   // uniform
    if (kr < eqtot || (a.cutoff != nullptr && !(a.cutoff_any && all_ties))) {
        block_scan(eqc, eqb, 0);
    } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q) eqb[q] = 0;
        kr = 0xFFFFFFFFu;   // every key equal to tau is selected
    }
    if (a.idx != nullptr) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            selc[q] = gtc[q] + (kr > eqb[q] ? min(eqc[q], kr - eqb[q]) : 0u);
        block_scan(selc, selb, 1);
    } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q) selb[q] = 0;
    }

    // Index list and cutoff (optional outputs): a separate pass behind one
    // uniform branch, so the common path carries no per-entry scatter.
    if (a.cutoff_any && all_ties && a.cutoff != nullptr && tid == 0) a.cutoff[r] = 0x7FFFFFFF;
    if (a.idx != nullptr || (a.cutoff != nullptr && !(a.cutoff_any && all_ties))) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (!run_valid(q)) continue;
            const int64_t j0 = (int64_t)q * CS + V * tid;
            uint32_t er = eqb[q], sp = selb[q];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const uint32_t kk = key[q * V + e];
                const bool gt = k > 0 && kk > tau;
                const bool eq = k > 0 && kk == tau;
                const bool sel = gt || (eq && er < kr);
                if (sel && sp < (uint32_t)k && a.idx != nullptr)
                    a.idx[(int64_t)r * a.idx_stride + sp] = (int32_t)(j0 + e);
                if (eq && er + 1 == kr && a.cutoff != nullptr) a.cutoff[r] = (int32_t)(j0 + e + 1);
                er += eq ? 1u : 0u;
                sp += sel ? 1u : 0u;
            }
        }
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        if (!run_valid(q)) continue;
        const int64_t j0 = (int64_t)q * CS + V * tid;
        uint32_t er = eqb[q];
        uint32_t mbits[(V + 3) / 4];
#pragma unroll
        for (int w = 0; w < (V + 3) / 4; ++w) mbits[w] = 0;
        uint32_t xsv[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const uint32_t kk = key[q * V + e];
            const bool gt = k > 0 && kk > tau;      // valid run: no invalid keys here
            const bool eq = k > 0 && kk == tau;
            const bool sel = gt || (eq && er < kr);
            mbits[e / 4] |= (sel ? 1u : 0u) << (8 * (e % 4));
            uint32_t xv = 0;
            if constexpr (XK == XS_F32) {
                float f = 0.0f;
                if constexpr (KK == KEY_F32) f = __uint_as_float(raw[q * V + e]);
                else if constexpr (KK == KEY_BF16) f = __uint_as_float(raw[q * V + e] << 16);
                else f = (float)(int32_t)raw[q * V + e];
                xv = sel ? __float_as_uint(f) : 0u;
            } else if constexpr (XK == XS_BF16) {
                xv = sel ? (raw[q * V + e] & 0xFFFFu) : 0u;
            } else if constexpr (XK == XS_I8) {
                xv = sel ? (raw[q * V + e] & 0xFFu) : 0u;
            }
            xsv[e] = xv;
            er += eq ? 1u : 0u;
        }
        if (a.mask != nullptr) {
            uint8_t* mp = a.mask + row0 + j0;
            if constexpr (V == 4) *reinterpret_cast<uint32_t*>(mp) = mbits[0];
            else if constexpr (V == 8) *reinterpret_cast<uint2*>(mp) = make_uint2(mbits[0], mbits[1]);
            else *reinterpret_cast<uint4*>(mp) = make_uint4(mbits[0], mbits[1], mbits[2], mbits[3]);
        }
        if constexpr (XK == XS_F32) {
            if (a.xs != nullptr) {
                float* xp = reinterpret_cast<float*>(a.xs) + row0 + j0;
#pragma unroll
                for (int e = 0; e < V; e += 4)
                    *reinterpret_cast<uint4*>(xp + e) = make_uint4(xsv[e], xsv[e + 1], xsv[e + 2], xsv[e + 3]);
            }
            if (a.frag != nullptr) {
                // Entries j0 .. j0 + V - 1 lie in one 8-entry chunk (V = 4 or
                // 8, j0 % V == 0): chunk (j0 % 32) / 8 of row group j0 / 32,
                // the record slot of token r % 16.
                uint32_t hi[V / 2], lo[V / 2];
#pragma unroll
                for (int e = 0; e < V; e += 2) {
                    const float c0 = __uint_as_float(xsv[e]), c1 = __uint_as_float(xsv[e + 1]);
                    const uint32_t h0 = frag_bf16_rne(c0), h1 = frag_bf16_rne(c1);
                    hi[e / 2] = h0 | (h1 << 16);
                    lo[e / 2] = frag_bf16_rne(c0 - __uint_as_float(h0 << 16)) |
                                (frag_bf16_rne(c1 - __uint_as_float(h1 << 16)) << 16);
                }
                const int64_t slot = ((int64_t)(r / 16) * a.frag_groups + j0 / 32) * 128 +
                                     16 * ((j0 % 32) / 8) + r % 16;
                char* base = reinterpret_cast<char*>(a.frag) + slot * 16 + (j0 % 8) * 2;
                if constexpr (V == 8) {
                    *reinterpret_cast<uint4*>(base) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                    if (a.frag_lo)
                        *reinterpret_cast<uint4*>(base + 64 * 16) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
                } else {
                    *reinterpret_cast<uint2*>(base) = make_uint2(hi[0], hi[1]);
                    if (a.frag_lo) *reinterpret_cast<uint2*>(base + 64 * 16) = make_uint2(lo[0], lo[1]);
                }
            }
        } else if constexpr (XK == XS_BF16) {
            if (a.xs != nullptr) {
                uint16_t* xp = reinterpret_cast<uint16_t*>(a.xs) + row0 + j0;   // V == 8
                *reinterpret_cast<uint4*>(xp) =
                    make_uint4(xsv[0] | (xsv[1] << 16), xsv[2] | (xsv[3] << 16),
                               xsv[4] | (xsv[5] << 16), xsv[6] | (xsv[7] << 16));
            }
        } else if constexpr (XK == XS_I8) {
            if (a.xs != nullptr) {
                int8_t* xp = reinterpret_cast<int8_t*>(a.xs) + row0 + j0;      // V == 4
                *reinterpret_cast<uint32_t*>(xp) = xsv[0] | (xsv[1] << 8) | (xsv[2] << 16) | (xsv[3] << 24);
            }
        }
    }
    if (tid == 0) {
        if (a.tau != nullptr) a.tau[r] = tau;
        if (k == 0 && a.cutoff != nullptr) a.cutoff[r] = 0;
        if (a.count != nullptr) a.count[r] = (int32_t)k;
    }
}

// Vectorised kernel with block size B, runs per thread chosen from the row length.
template <int B, int KK, int XK>
hipError_t launch_vec(int64_t rows, const TopkArgs& a, hipStream_t stream) {
    // At most 32 keys per thread (NQ * V <= 32): more would spill scalar
    // registers in the unrolled per-entry loops.
    constexpr int V = VecOf<KK>::V, CS = V * B;
    constexpr int kRowNQ = 16384 / CS > 0 ? 16384 / CS : 1;     // rows of at most 16384
    constexpr int kMaxNQ = 32 / V < kRowNQ ? 32 / V : kRowNQ;
    const dim3 grid((unsigned)rows), block(B);
    const int64_t nq = (a.d + CS - 1) / CS;
    if (nq <= 1) topk_vec_kernel<B, 1, KK, XK><<<grid, block, 0, stream>>>(a);
    else if (nq <= 2) topk_vec_kernel<B, 2, KK, XK><<<grid, block, 0, stream>>>(a);
    else if constexpr (kMaxNQ >= 4) {
        if (nq <= 3) topk_vec_kernel<B, 3, KK, XK><<<grid, block, 0, stream>>>(a);
        else if (nq <= 4) topk_vec_kernel<B, 4, KK, XK><<<grid, block, 0, stream>>>(a);
        else if constexpr (kMaxNQ >= 8) {
            if (nq <= 8) topk_vec_kernel<B, 8, KK, XK><<<grid, block, 0, stream>>>(a);
            else return hipErrorInvalidValue;
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int NT, int KK, int XK>
hipError_t launch_kkx(int64_t rows, const TopkArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)rows), block(NT);
    constexpr int R = 256;   // the register-resident scalar kernel runs 4 waves
    constexpr int V = VecOf<KK>::V;
    if (a.d % V == 0 && a.d <= 16384) {
        // Few rows (decode): 16 waves per row hide each other's latencies;
        // many rows: 4 waves per row and many rows per CU, unless a row needs
        // more than 32 keys per thread.
        if (rows <= 64 && a.d >= 1024 * V) return launch_vec<1024, KK, XK>(rows, a, stream);
        if (rows <= 64 && a.d >= 512 * V) return launch_vec<512, KK, XK>(rows, a, stream);
        if (a.d <= 256 * 32) return launch_vec<256, KK, XK>(rows, a, stream);
        return launch_vec<512, KK, XK>(rows, a, stream);
    }
    if (a.d <= 4 * R) {
        topk_reg_kernel<R, 4, KK, XK><<<grid, dim3(R), 0, stream>>>(a);
    } else if (a.d <= 8 * R) {
        topk_reg_kernel<R, 8, KK, XK><<<grid, dim3(R), 0, stream>>>(a);
    } else if (a.d <= 16 * R) {
        topk_reg_kernel<R, 16, KK, XK><<<grid, dim3(R), 0, stream>>>(a);
    } else if (a.d <= 32 * R) {
        topk_reg_kernel<R, 32, KK, XK><<<grid, dim3(R), 0, stream>>>(a);
    } else if (a.d <= 48 * R) {
        topk_reg_kernel<R, 48, KK, XK><<<grid, dim3(R), 0, stream>>>(a);
    } else if (a.d <= 64 * R) {
        topk_reg_kernel<R, 64, KK, XK><<<grid, dim3(R), 0, stream>>>(a);
    } else if (a.d <= kStageMaxD) {
        size_t smem = (size_t)a.d * sizeof(uint32_t);
        topk_rows_kernel<NT, KK, XK, true><<<grid, block, smem, stream>>>(a);
    } else {
        topk_rows_kernel<NT, KK, XK, false><<<grid, block, 0, stream>>>(a);
    }
    return hipGetLastError();
}

template <int NT>
hipError_t launch_nt(int key_kind, int xs_kind, int64_t rows, const TopkArgs& a,
                     hipStream_t stream) {
    switch (key_kind) {
    case KEY_F32:
        if (xs_kind == XS_NONE) return launch_kkx<NT, KEY_F32, XS_NONE>(rows, a, stream);
        if (xs_kind == XS_F32) return launch_kkx<NT, KEY_F32, XS_F32>(rows, a, stream);
        break;
    case KEY_BF16:
        if (xs_kind == XS_NONE) return launch_kkx<NT, KEY_BF16, XS_NONE>(rows, a, stream);
        if (xs_kind == XS_F32) return launch_kkx<NT, KEY_BF16, XS_F32>(rows, a, stream);
        if (xs_kind == XS_BF16) return launch_kkx<NT, KEY_BF16, XS_BF16>(rows, a, stream);
        break;
    case KEY_I8:
        if (xs_kind == XS_NONE) return launch_kkx<NT, KEY_I8, XS_NONE>(rows, a, stream);
        break;
    case KEY_Q8:
        if (xs_kind == XS_I8) return launch_kkx<NT, KEY_Q8, XS_I8>(rows, a, stream);
        if (xs_kind == XS_NONE) return launch_kkx<NT, KEY_Q8, XS_NONE>(rows, a, stream);
        break;
    }
    return hipErrorInvalidValue;
}

__global__ void zero_i32_kernel(int32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

}  // namespace

bool topk_xform_supported(int64_t d) { return d % 4 == 0 && d <= 16384; }

// ---------------------------------------------------------------------------
// Top-k descriptor of a row of fp32 values by magnitude (the FFN
// intermediate; Turbo Sparse summary, Eq. 3-4: the top-k% of h by |h| before
// W_down), when neither the index list nor the sparsified row is wanted: the
// next launch applies (tau, cutoff) itself.  One workgroup per row, NQ runs
// of 4 entries per thread; rowsel::select_desc31 does the rest.  1024
// threads: the passes over the keys are chains of short dependent steps, and
// four wavefronts per SIMD hide each other's waits (with 256 threads, 44 keys
// each, the same search took 5.5 us instead of 3.2).
// ---------------------------------------------------------------------------
constexpr int kDescNT = 1024;

template <int NQ>
__global__ __launch_bounds__(kDescNT) void desc31_kernel(const float* x, int64_t rows, int64_t d,
                                                         int64_t k, uint32_t* desc) {
    __shared__ rowsel::Sel31Lds<NQ, kDescNT / 64> L;
    const int r = blockIdx.x, tid = threadIdx.x;
    rowsel::sel31_clear<kDescNT, NQ>(L, tid);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(x + (int64_t)r * d), (short)0, (int)(d * 4), 0x00020000);
    uint32_t key[4 * NQ];   // past the row end (d % 4 == 0) the loads read 0
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
            rs, (uint32_t)((q * 4 * kDescNT + 4 * tid) * 4), 0, 0);
        key[4 * q] = v.x & 0x7FFFFFFFu; key[4 * q + 1] = v.y & 0x7FFFFFFFu;
        key[4 * q + 2] = v.z & 0x7FFFFFFFu; key[4 * q + 3] = v.w & 0x7FFFFFFFu;
    }
    // (an empty asm per key: the compiler would otherwise keep the loaded
    // words as well, to recompute each key where it is used)
#pragma unroll
    for (int i = 0; i < 4 * NQ; ++i) asm volatile("" : "+v"(key[i]));
    __syncthreads();
    uint32_t tau, cut;
    rowsel::select_desc31<kDescNT, NQ>(key, d, k, L, tid, tau, cut);
    if (tid == 0) { desc[r] = tau; desc[rows + r] = cut; }
}

hipError_t launch_desc31(const float* x, int64_t rows, int64_t d, int64_t k, uint32_t* desc,
                         hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    if (!desc31_supported(d)) return hipErrorInvalidValue;
    const int nq = (int)((d + 4 * kDescNT - 1) / (4 * kDescNT));
    const dim3 grid((unsigned)rows), block(kDescNT);
    if (nq <= 1) desc31_kernel<1><<<grid, block, 0, stream>>>(x, rows, d, k, desc);
    else if (nq <= 2) desc31_kernel<2><<<grid, block, 0, stream>>>(x, rows, d, k, desc);
    else if (nq <= 3) desc31_kernel<3><<<grid, block, 0, stream>>>(x, rows, d, k, desc);
    else desc31_kernel<4><<<grid, block, 0, stream>>>(x, rows, d, k, desc);
    return hipGetLastError();
}

namespace {

// Rows of bf16 x whose only output is X (.) M: in bf16 for many rows (the
// operand of the dense MFMA paths), in fp32 for a few (the decode FFN's
// gathers); one workgroup of NT threads per row, E entries per thread.  The top-k of the 15-bit magnitude keys comes from two LDS
// histogram levels (8 high bits, then the 7 low bits of the boundary bin;
// ties to the lower index, Q-Sparse news article, section "Sparsification
// with the Top-K function"), without the candidate lists and digit loops of
// the general kernel; then each thread writes its run of X (.) M (bf16, or
// fp32 with F32), after the launch's side jobs (clear_side_buffers).
constexpr int kS15NT = 256;

template <int NT, int E, bool F32>
__global__ __launch_bounds__(NT) void select15_xs_kernel(TopkArgs a) {
    __shared__ rowsel::Sel15Lds<1, NT / 64> L;
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int d = (int)a.d;
    const int nvalid = d - tid * E;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(reinterpret_cast<const void*>(reinterpret_cast<const uint16_t*>(a.x) + row * d)),
        (short)0, d * 2, 0x00020000);
    uint32_t xr16[E / 2];   // bf16 pairs (entry 2i in the low half)
#pragma unroll
    for (int q = 0; q < E / 8; ++q) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(xr, (uint32_t)((tid * E + 8 * q) * 2), 0, 0);
        xr16[4 * q] = v.x; xr16[4 * q + 1] = v.y; xr16[4 * q + 2] = v.z; xr16[4 * q + 3] = v.w;
    }
    clear_side_buffers<NT>(a, (int)row, tid);
    for (int i = tid; i < (int)(sizeof(L) / 4); i += NT) reinterpret_cast<uint32_t*>(&L)[i] = 0;
    uint32_t key[1][E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        key[0][e] = e < nvalid ? (xr16[e / 2] >> (16 * (e % 2))) & 0x7FFFu : sel::kInvalid;
    __syncthreads();
    uint32_t selm[1];
    rowsel::select15_masks<NT, 1, E>(key, 1, a.k, L, tid, selm);
#pragma unroll
    for (int q = 0; q < E / 8; ++q) {
        if (tid * E + 8 * q >= d) break;   // (d % 8 == 0: whole runs)
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 8 * q + 2 * i;
            const uint32_t lo = (selm[0] >> e) & 1u ? 0x0000FFFFu : 0u;
            const uint32_t hi = (selm[0] >> (e + 1)) & 1u ? 0xFFFF0000u : 0u;
            w[i] = xr16[4 * q + i] & (lo | hi);
        }
        if constexpr (F32) {
            // bf16 -> fp32 is exact: the bits move to the high half.
            float* xs = reinterpret_cast<float*>(a.xs) + row * d + tid * E + 8 * q;
            *reinterpret_cast<uint4*>(xs) = make_uint4(w[0] << 16, w[0] & 0xFFFF0000u,
                                                       w[1] << 16, w[1] & 0xFFFF0000u);
            *reinterpret_cast<uint4*>(xs + 4) = make_uint4(w[2] << 16, w[2] & 0xFFFF0000u,
                                                           w[3] << 16, w[3] & 0xFFFF0000u);
        } else {
            uint16_t* xs = reinterpret_cast<uint16_t*>(a.xs) + row * d;
            *reinterpret_cast<uint4*>(xs + tid * E + 8 * q) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

}  // namespace

hipError_t launch_topk(int key_kind, int xs_kind, int64_t rows, const TopkArgs& a,
                       hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    // The elementwise map lives in the vector kernel, which takes exactly
    // these rows (fp32 keys, d % 4 == 0, d <= 16384).
    if (a.xform != XF_NONE &&
        (key_kind != KEY_F32 || !topk_xform_supported(a.d) || a.xform > XF_RELU2_GLU ||
         (a.xform == XF_RELU2_GLU && a.x2 == nullptr)))
        return hipErrorInvalidValue;
    if ((a.zero_rows != nullptr || a.zero_rows2 != nullptr) && a.zero_row_len % 4 != 0)
        return hipErrorInvalidValue;
    // Packed records: fp32 values of the vector kernel (d % 8 == 0 keeps every
    // run inside one 8-entry chunk).
    if (a.frag != nullptr &&
        (xs_kind != XS_F32 || (key_kind != KEY_F32 && key_kind != KEY_BF16) || a.d % 8 != 0 ||
         a.d > 16384 || a.frag_groups != (a.d + 31) / 32))
        return hipErrorInvalidValue;
    // Rows of bf16 keys whose only output is X (.) M (besides the side jobs):
    // the lean two-level selection.  Many rows written in bf16 (measured
    // against the general kernel on the 2048 x 4096 prefill rows): 256
    // threads per row; few rows written in fp32 (the 2-16 token decode FFN):
    // 512 threads per row, for latency.
    const bool lean = key_kind == KEY_BF16 && rows <= 0x7FFFFFFF && a.d % 8 == 0 &&
                      a.xs != nullptr && a.mask == nullptr && a.idx == nullptr &&
                      a.count == nullptr && a.tau == nullptr && a.cutoff == nullptr &&
                      a.xform == XF_NONE && a.frag == nullptr;
    if (lean && xs_kind == XS_BF16 && rows > 64 && a.d <= 16 * kS15NT &&
        a.zero_rows == nullptr && a.zero_rows2 == nullptr) {
        const dim3 g((unsigned)rows), b(kS15NT);
        if (a.d <= 8 * kS15NT) select15_xs_kernel<kS15NT, 8, false><<<g, b, 0, stream>>>(a);
        else select15_xs_kernel<kS15NT, 16, false><<<g, b, 0, stream>>>(a);
        return hipGetLastError();
    }
    if (lean && xs_kind == XS_F32 && rows <= 64 && a.d <= 16 * 512) {
        const dim3 g((unsigned)rows), b(512);
        if (a.d <= 8 * 512) select15_xs_kernel<512, 8, true><<<g, b, 0, stream>>>(a);
        else select15_xs_kernel<512, 16, true><<<g, b, 0, stream>>>(a);
        return hipGetLastError();
    }
    // Few rows (decode): one big workgroup per row; many rows: smaller ones.
    if (rows <= 64) return launch_nt<1024>(key_kind, xs_kind, rows, a, stream);
    return launch_nt<256>(key_kind, xs_kind, rows, a, stream);
}

hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    int blocks = (int)((n + 255) / 256);
    if (blocks > 1024) blocks = 1024;
    zero_i32_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(p, n);
    return hipGetLastError();
}

}  // namespace qs
