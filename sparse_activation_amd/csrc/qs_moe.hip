// Mixture-of-experts routing and combine for the dReLU MoE FFN.
//
// Turbo Sparse summary (blog.csdn.net), per-layer zero-activation passage:
// the MoE model activates 2 of its 8 experts per layer and, with dReLU, only
// ~15% of each expert's neurons, so ~3% of the layer's parameters are used
// per token.  The routing rule is not on the pages; the reading taken is the
// usual one for that model family: logits = x . W_router^T, the top_k logits
// of each token (ties to the lower expert index), softmax over the kept
// logits only.  The experts themselves run through the dReLU kernels with a
// (token, expert) pair per launch row; this file holds the router and the
// weighted sum of the pairs' outputs.
#include "qs_internal.h"

namespace qs {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Sum over the 64 lanes of a wavefront (fixed butterfly order).
__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

// Order-preserving map of a float to an unsigned key (larger float, larger key).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
    const uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// One workgroup of 8 wavefronts per token.  Wavefront w computes the logits
// of experts w, w + 8, ...: each lane loads its NCH runs of 8 features
// (features 512 i + 8 lane ..) of x and of the expert's router row at once,
// sums the products in run order, then the wavefront adds the lanes in a
// fixed butterfly.  Wavefront 0 then selects the experts with lane e holding
// logit e: top_k rounds of a wavefront max over (logit, lower index first),
// and the softmax over the chosen lanes.
template <int NCH>
__global__ __launch_bounds__(512) void moe_route_kernel(MoeRouteArgs a) {
    __shared__ float s_logit[64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t = blockIdx.x, d = a.d;
    const int E = a.n_experts, K = a.top_k;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.x + t * d), (short)0, (int)(d * 2), 0x00020000);
    u32x4 xv[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int64_t k = (int64_t)i * 512 + 8 * lane;
        xv[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, k < d ? (uint32_t)(k * 2) : 0x80000000u, 0, 0);
    }
    for (int e = wave; e < E; e += 8) {
        const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(a.wr + (int64_t)e * d), (short)0, (int)(d * 2), 0x00020000);
        u32x4 wv[NCH];
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int64_t k = (int64_t)i * 512 + 8 * lane;
            wv[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, k < d ? (uint32_t)(k * 2) : 0x80000000u, 0, 0);
        }
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s = __fmaf_rn(bf16_lo(xv[i][q]), bf16_lo(wv[i][q]), s);
                s = __fmaf_rn(bf16_hi(xv[i][q]), bf16_hi(wv[i][q]), s);
            }
        s = wave_sum64(s);
        if (lane == 0) s_logit[e] = s;
    }
    __syncthreads();
    if (wave != 0) return;
    const bool valid = lane < E;
    const float lg = valid ? s_logit[lane] : 0.0f;
    if (valid && a.logits != nullptr) a.logits[t * E + lane] = lg;
    // key: logit order in the high word, then the lower lane wins
    const uint64_t key = valid ? ((uint64_t)f32_order_key(lg) << 32) | (uint32_t)(63 - lane) : 0;
    bool chosen = false;
    float mx = 0.0f;
    for (int j = 0; j < K; ++j) {
        uint64_t best = chosen ? 0 : key;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const uint64_t o = ((uint64_t)(uint32_t)__shfl_xor((int)(best >> 32), m, 64) << 32) |
                               (uint32_t)__shfl_xor((int)(best & 0xFFFFFFFFu), m, 64);
            best = o > best ? o : best;
        }
        const int win = 63 - (int)(best & 0xFFFFFFFFu);
        if (lane == win) chosen = true;
        if (j == 0) mx = __shfl(lg, win, 64);
    }
    const float p = chosen ? expf(lg - mx) : 0.0f;
    const float sum = wave_sum64(p);
    const uint64_t sel = __ballot(chosen);
    if (chosen) {
        const int pos = __popcll(sel & ((uint64_t(1) << lane) - 1));
        const int64_t q = t * K + pos;
        const float wq = p / sum;
        a.pair_token[q] = (int32_t)t;
        a.pair_expert[q] = lane;
        a.pair_weight[q] = wq;
        if (a.out_experts != nullptr) a.out_experts[q] = lane;
        if (a.out_weights != nullptr) a.out_weights[q] = wq;
    }
}

// y[t, c] = sum over j < top_k of weight[t, j] * ypair[t * top_k + j, c], in
// j order; four columns per thread.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ ypair,
                                                          const float* __restrict__ w,
                                                          int64_t rows, int top_k, int64_t d,
                                                          void* __restrict__ y, int y_bf16) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per = d / 4;
    if (i >= rows * per) return;
    const int64_t t = i / per, c = (i % per) * 4;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < top_k; ++j) {
        const float wj = w != nullptr ? w[t * top_k + j] : 1.0f;
        const float4 v = *reinterpret_cast<const float4*>(ypair + (t * top_k + j) * d + c);
        acc[0] = __fmaf_rn(wj, v.x, acc[0]);
        acc[1] = __fmaf_rn(wj, v.y, acc[1]);
        acc[2] = __fmaf_rn(wj, v.z, acc[2]);
        acc[3] = __fmaf_rn(wj, v.w, acc[3]);
    }
    if (y_bf16) {
        uint16_t* o = reinterpret_cast<uint16_t*>(y) + t * d + c;
        const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
        *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
    } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + t * d + c) =
            make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
}

// One workgroup: expert e's pairs go to list[e * pairs + slot] with their
// tokens in tok[e * pairs + slot], slots taken with LDS atomics, and the
// counts to count[e].
__global__ __launch_bounds__(256) void moe_group_kernel(const int32_t* __restrict__ pair_expert,
                                                        const int32_t* __restrict__ pair_token,
                                                        int64_t pairs, int n_experts,
                                                        int32_t* __restrict__ count,
                                                        int32_t* __restrict__ list,
                                                        int32_t* __restrict__ tok) {
    __shared__ uint32_t s_cnt[64];
    const int tid = threadIdx.x;
    if (tid < 64) s_cnt[tid] = 0;
    __syncthreads();
    for (int64_t q = tid; q < pairs; q += 256) {
        const int e = pair_expert[q];
        const int64_t slot = atomicAdd(&s_cnt[e], 1u);
        list[e * pairs + slot] = (int32_t)q;
        tok[e * pairs + slot] = pair_token[q];
    }
    __syncthreads();
    if (tid < n_experts) count[tid] = (int32_t)s_cnt[tid];
}

}  // namespace

hipError_t launch_moe_group(const int32_t* pair_expert, const int32_t* pair_token, int64_t pairs,
                            int n_experts, int32_t* count, int32_t* list, int32_t* tok,
                            hipStream_t stream) {
    if (pairs <= 0) return hipSuccess;
    if (n_experts < 1 || n_experts > 64) return hipErrorInvalidValue;
    moe_group_kernel<<<dim3(1), dim3(256), 0, stream>>>(pair_expert, pair_token, pairs, n_experts,
                                                        count, list, tok);
    return hipGetLastError();
}

hipError_t launch_moe_route(const MoeRouteArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    if (a.n_experts < 1 || a.n_experts > 64 || a.top_k < 1 || a.top_k > a.n_experts || a.d % 8 != 0)
        return hipErrorInvalidValue;
    if (a.d > 8192) return hipErrorInvalidValue;
    const int nch = (int)((a.d + 511) / 512);
    const dim3 grid((unsigned)a.rows), block(512);
    if (nch <= 2) moe_route_kernel<2><<<grid, block, 0, stream>>>(a);
    else if (nch <= 4) moe_route_kernel<4><<<grid, block, 0, stream>>>(a);
    else if (nch <= 8) moe_route_kernel<8><<<grid, block, 0, stream>>>(a);
    else moe_route_kernel<16><<<grid, block, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_moe_combine(const float* ypair, const float* pair_weight, int64_t rows,
                              int top_k, int64_t d, void* y, int y_bf16, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    if (d % 4 != 0) return hipErrorInvalidValue;
    const int64_t n = rows * (d / 4);
    moe_combine_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(
        ypair, pair_weight, rows, top_k, d, y, y_bf16);
    return hipGetLastError();
}

}  // namespace qs
