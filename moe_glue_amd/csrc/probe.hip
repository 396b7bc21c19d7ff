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

// Streams with a given read:write mix, as independent read and write waves:
// in each cycle of reads + writes waves the first `reads` each load U KiB of
// src (U vectors per lane, every access of a wave one contiguous KiB) and the
// others each store U KiB to dst.  Nothing a wave writes depends on a read,
// so the figure is what HBM gives that mix, not the latency of a kernel's
// load-then-store chain.  The loaded values only feed a store that never
// happens (it keeps the loads).
template <int TH, int U>
__global__ __launch_bounds__(TH) void mix_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                       uint32_t waves, uint32_t reads, uint32_t writes) {
    const uint32_t g = blockIdx.x * (TH / kThreads) + threadIdx.x / kThreads;
    if (g >= waves) return;
    const uint32_t l = threadIdx.x % kThreads;
    const uint32_t cyc = g / (reads + writes), pos = g % (reads + writes);
    if (pos < reads) {
        const size_t base = ((size_t)cyc * reads + pos) * kThreads * U;
        u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= load_stream(src + base + (size_t)u * kThreads + l);
        if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u && acc[2] == 0x85EBCA6Bu && acc[3] == g)
            store_stream(dst + l, acc);  // never for the probe's data
    } else {
        const size_t base = ((size_t)cyc * writes + (pos - reads)) * kThreads * U;
        const u32x4 v = {g, l, cyc, pos};
#pragma unroll
        for (int u = 0; u < U; ++u) store_stream(dst + base + (size_t)u * kThreads + l, v);
    }
}

template <int TH, int U>
void launch_mix(const void* src, void* dst, uint32_t waves, uint32_t reads, uint32_t writes, hipStream_t stream) {
    const uint32_t blocks = (waves + TH / kThreads - 1) / (TH / kThreads);
    mix_probe_kernel<TH, U><<<dim3(blocks), TH, 0, stream>>>(static_cast<const u32x4*>(src),
                                                             static_cast<u32x4*>(dst), waves, reads, writes);
}

}  // namespace

hipError_t launch_mix_probe(const void* src, void* dst, uint32_t cycles, uint32_t reads, uint32_t writes,
                            int vectors_per_lane, int threads, hipStream_t stream) {
    const uint32_t waves = cycles * (reads + writes);
    switch (threads * 8 + vectors_per_lane) {
        case 64 * 8 + 1: launch_mix<64, 1>(src, dst, waves, reads, writes, stream); break;
        case 64 * 8 + 2: launch_mix<64, 2>(src, dst, waves, reads, writes, stream); break;
        case 64 * 8 + 4: launch_mix<64, 4>(src, dst, waves, reads, writes, stream); break;
        case 256 * 8 + 1: launch_mix<256, 1>(src, dst, waves, reads, writes, stream); break;
        case 256 * 8 + 2: launch_mix<256, 2>(src, dst, waves, reads, writes, stream); break;
        case 256 * 8 + 4: launch_mix<256, 4>(src, dst, waves, reads, writes, stream); break;
        case 1024 * 8 + 1: launch_mix<1024, 1>(src, dst, waves, reads, writes, stream); break;
        case 1024 * 8 + 2: launch_mix<1024, 2>(src, dst, waves, reads, writes, stream); break;
        default: launch_mix<1024, 4>(src, dst, waves, reads, writes, stream); break;
    }
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
