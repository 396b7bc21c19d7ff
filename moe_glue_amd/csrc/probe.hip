// A plain streaming copy, 16 bytes per lane, used as the measuring stick for
// achievable HBM bandwidth and to calibrate the traffic counters.  It is not
// part of the MoE path.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

// One wave per workgroup: the fastest plain copy measured on this part
// (1 GiB each way: 6.68 TB/s against 6.44 with 256 lanes).
constexpr int kThreads = 64;
constexpr int kU = 1;

__global__ __launch_bounds__(kThreads) void copy_probe_kernel(const u32x4* __restrict__ src,
                                                              u32x4* __restrict__ dst, size_t n) {
    const size_t base = (size_t)blockIdx.x * (kThreads * kU) + threadIdx.x;
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const size_t i = base + (size_t)u * kThreads;
        if (i < n) v[u] = load_stream(src + i);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const size_t i = base + (size_t)u * kThreads;
        if (i < n) store_stream(dst + i, v[u]);
    }
}

}  // namespace

hipError_t launch_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    const size_t n = bytes / 16;
    const size_t blocks = (n + kThreads * kU - 1) / (kThreads * kU);
    copy_probe_kernel<<<dim3((unsigned)blocks), kThreads, 0, stream>>>(static_cast<const u32x4*>(src),
                                                                      static_cast<u32x4*>(dst), n);
    return hipGetLastError();
}

}  // namespace moe
