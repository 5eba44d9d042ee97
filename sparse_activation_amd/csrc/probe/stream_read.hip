// Bandwidth reference for measurements (libqs_probe.so, not part of libqs.so
// or its ABI): a plain streaming read of a device buffer.  The gather
// kernels' HBM throughput is reported against the published peak and against
// what this read reaches on the same number of bytes, the practical ceiling of
// a kernel that size.
//
//   int qsprobe_stream_read(const void* src, size_t bytes, uint32_t* sink,
//                           void* stream)
//     src    device, 16-byte aligned; bytes % 16 == 0.
//     sink   device u32, written only if the checksum of the data equals a
//            fixed constant (never in practice).
//     Returns 0, 1 (bad argument) or 2 (HIP launch error).  Asynchronous on
//     `stream` (a hipStream_t).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace qs {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeWG = 1024;   // workgroups of 256 threads
constexpr int kProbeNF = 16;     // 16-byte loads in flight per lane

// Workgroup b reads the b-th contiguous chunk of the buffer; every lane keeps
// kProbeNF loads in flight.  The values are folded into a checksum that is
// stored only if it equals a constant no real input produces by design, so
// the loads stay live without a store per workgroup.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* p, size_t n16, uint32_t* sink) {
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b = (size_t)blockIdx.x * per;
    const size_t e = b + per < n16 ? b + per : n16;
    uint32_t acc = 0;
    size_t i = b + threadIdx.x;
    for (; i + (size_t)(kProbeNF - 1) * 256 < e; i += (size_t)kProbeNF * 256) {
        u32x4 v[kProbeNF];
#pragma unroll
        for (int u = 0; u < kProbeNF; ++u) v[u] = p[i + (size_t)u * 256];
#pragma unroll
        for (int u = 0; u < kProbeNF; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < e; i += 256) {
        const u32x4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace
}  // namespace qs

extern "C" int qsprobe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (src == nullptr || sink == nullptr) return 1;
    if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0) return 1;
    if (bytes == 0) return 0;
    qs::stream_read_kernel<<<dim3(qs::kProbeWG), dim3(256), 0, (hipStream_t)stream>>>(
        static_cast<const qs::u32x4*>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
