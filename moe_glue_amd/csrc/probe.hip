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

// Streams with a given read:write mix: lane i of wave w reads `reads`
// vectors of its wave's block of src and writes `writes` vectors (all built
// from what it read) to its block of dst, every access of a wave one
// contiguous 1 KiB.  No kernel of the path is this plain; it tells what
// HBM gives a stream with a path kernel's mix of reads and writes.
__global__ __launch_bounds__(kThreads) void mix_probe_kernel(const u32x4* __restrict__ src,
                                                             u32x4* __restrict__ dst, uint32_t lanes,
                                                             uint32_t reads, uint32_t writes) {
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= lanes) return;
    const size_t block = (size_t)(i / kThreads) * kThreads;
    const uint32_t l = i % kThreads;
    u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll 8
    for (uint32_t r = 0; r < reads; ++r) acc ^= load_stream(src + block * reads + (size_t)r * kThreads + l);
#pragma unroll 8
    for (uint32_t w = 0; w < writes; ++w) {
        u32x4 v = acc;
        v[0] += w;
        store_stream(dst + block * writes + (size_t)w * kThreads + l, v);
    }
}

}  // namespace

hipError_t launch_mix_probe(const void* src, void* dst, uint32_t lanes, uint32_t reads, uint32_t writes,
                            hipStream_t stream) {
    const uint32_t blocks = (lanes + kThreads - 1) / kThreads;
    mix_probe_kernel<<<dim3(blocks), kThreads, 0, stream>>>(static_cast<const u32x4*>(src), static_cast<u32x4*>(dst),
                                                            lanes, reads, writes);
    return hipGetLastError();
}

hipError_t launch_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    const size_t n = bytes / 16;
    const size_t blocks = (n + kThreads * kU - 1) / (kThreads * kU);
    copy_probe_kernel<<<dim3((unsigned)blocks), kThreads, 0, stream>>>(static_cast<const u32x4*>(src),
                                                                      static_cast<u32x4*>(dst), n);
    return hipGetLastError();
}

}  // namespace moe
