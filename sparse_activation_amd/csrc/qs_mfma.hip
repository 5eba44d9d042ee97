// MFMA kernels (gfx950): the masked dense GEMM for large token batches and
// the dReLU gate/up projection, plus the nonzero compaction of the FFN
// intermediate.
#include "qs_internal.h"

namespace qs {
namespace {

__device__ __forceinline__ uint32_t popc_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
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

}  // namespace

hipError_t launch_nonzero_lists(const float* h, int64_t rows, int64_t n, int32_t* idx,
                                int32_t* cnt, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    nonzero_lists_kernel<<<dim3((unsigned)rows), dim3(256), 0, stream>>>(h, n, idx, cnt);
    return hipGetLastError();
}

hipError_t launch_masked_gemm(const MfmaArgs&, hipStream_t) { return hipErrorNotSupported; }

hipError_t launch_drelu_gate_up(const DreluArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace qs
