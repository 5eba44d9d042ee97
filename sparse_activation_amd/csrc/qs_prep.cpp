// Offline weight preparation for the quantised path (host code, not timed).
//
// Q-Sparse news article (zxwl-tech.com), section "Sparsification with the
// Top-K function": for 1-bit (ternary, BitNet b1.58) weights the quantiser
// scales by alpha, the mean absolute value of the weight tensor.
//
// alpha is computed from the exact sum of |w|: every binary32 |w| is an
// integer mantissa times a power of two, so the mantissas are summed exactly
// per exponent in 64-bit bins, the bins are carried into one exact binary
// number, and that number is rounded once to binary64 (nearest, ties to
// even).  Then alpha = fl32(fl64(sum) / n).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/qs.h"
#include "qs_error.h"

namespace {

// Correctly rounded binary64 value of sum_i |w_i| for binary32 inputs.
double exact_abs_sum(const float* w, int64_t n) {
    // |w| = m * 2^(E - 150), E = max(biased exponent, 1), m < 2^24.
    std::vector<int64_t> bins(256, 0);
    for (int64_t i = 0; i < n; ++i) {
        uint32_t b;
        std::memcpy(&b, &w[i], 4);
        b &= 0x7FFFFFFFu;
        const uint32_t e = b >> 23;
        uint32_t m = b & 0x7FFFFFu;
        if (e != 0) m |= 0x800000u;
        bins[e == 0 ? 1 : e] += m;
    }
    // Carry into bits: bit p has weight 2^(p - 150).
    std::vector<uint8_t> bits;
    bits.reserve(400);
    int64_t carry = 0;
    for (int p = 0; p < 256 || carry != 0; ++p) {
        if (p < 256) carry += bins[p];
        bits.push_back((uint8_t)(carry & 1));
        carry >>= 1;
    }
    int hi = (int)bits.size() - 1;
    while (hi >= 0 && bits[hi] == 0) --hi;
    if (hi < 0) return 0.0;
    // Keep 53 significant bits, round to nearest, ties to even.
    uint64_t mant = 0;
    const int lo = hi - 52;
    for (int p = hi; p >= lo; --p) mant = (mant << 1) | (p >= 0 ? bits[p] : 0);
    if (lo > 0) {
        const int round_bit = bits[lo - 1];
        bool sticky = false;
        for (int p = lo - 2; p >= 0 && !sticky; --p) sticky = bits[p] != 0;
        if (round_bit && (sticky || (mant & 1))) ++mant;
    }
    // mant holds bits hi..lo (bits below 0 read as zero): value = mant * 2^(lo - 150)
    return std::ldexp((double)mant, lo - 150);
}

}  // namespace

extern "C" {

qs_status qs_ternarize(const float* w_host, int64_t n_out, int64_t d_in, int8_t* t_host,
                       float* alpha) {
    if (!w_host || !t_host || !alpha || n_out <= 0 || d_in <= 0)
        return qs::set_error(QS_ERR_INVALID_ARG, "qs_ternarize: NULL pointer or empty shape");
    const int64_t n = n_out * d_in;
    const double sum = exact_abs_sum(w_host, n);
    const float a = (float)(sum / (double)n);
    const float den = a + 1e-5f;
    for (int64_t i = 0; i < n; ++i) {
        float q = std::rint(w_host[i] / den);
        if (q > 1.0f) q = 1.0f;
        if (q < -1.0f) q = -1.0f;
        t_host[i] = (int8_t)q;
    }
    *alpha = a;
    return qs::set_error(QS_OK, "");
}

qs_status qs_pack_ternary(const int8_t* t_host, int64_t n_out, int64_t d_in, uint8_t* packed_host) {
    if (!t_host || !packed_host || n_out <= 0 || d_in <= 0)
        return qs::set_error(QS_ERR_INVALID_ARG, "qs_pack_ternary: NULL pointer or empty shape");
    if (n_out % 4 != 0)
        return qs::set_error(QS_ERR_UNSUPPORTED, "qs_pack_ternary: n_out must be a multiple of 4");
    const int64_t nb = n_out / 4;
    for (int64_t i = 0; i < n_out * d_in; ++i)
        if (t_host[i] < -1 || t_host[i] > 1)
            return qs::set_error(QS_ERR_INVALID_ARG, "qs_pack_ternary: values must be in {-1, 0, 1}");
    for (int64_t j = 0; j < d_in; ++j) {
        for (int64_t c4 = 0; c4 < nb; ++c4) {
            uint32_t byte = 0;
            for (int i = 0; i < 4; ++i) {
                const int8_t t = t_host[(c4 * 4 + i) * d_in + j];
                byte |= ((uint32_t)t & 3u) << (2 * i);   // 2-bit two's complement
            }
            packed_host[j * nb + c4] = (uint8_t)byte;
        }
    }
    return qs::set_error(QS_OK, "");
}

}  // extern "C"
