// Plain streaming read of a device buffer: the machine's read rate that the
// decode (one pass over its packed K/V cache per call) is measured against.
// Each of the G workgroups of 256 threads reads one contiguous range with
// 16-byte loads, four in flight per thread; each wave writes the XOR of what
// it read to one word of the sink so that no load can be removed.
#include "qkv_internal.hpp"
#include "qkv_measure.h"

namespace qkv {

namespace {

constexpr int kReadThreads = 256;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* __restrict__ p, uint64_t n16,
                                                                    uint64_t per_wg, uint32_t* __restrict__ sink) {
    const uint64_t b = (uint64_t)blockIdx.x * per_wg;
    const uint64_t e = b + per_wg < n16 ? b + per_wg : n16;
    constexpr uint64_t T = kReadThreads;
    uint32_t acc = 0;
    uint64_t i = b + threadIdx.x;
    for (; i + 3 * T < e; i += 4 * T) {
        const uint4 x0 = p[i], x1 = p[i + T], x2 = p[i + 2 * T], x3 = p[i + 3 * T];
        acc ^= x0.x ^ x0.y ^ x0.z ^ x0.w ^ x1.x ^ x1.y ^ x1.z ^ x1.w ^ x2.x ^ x2.y ^ x2.z ^ x2.w ^ x3.x ^ x3.y ^
               x3.z ^ x3.w;
    }
    for (; i < e; i += T) {
        const uint4 x = p[i];
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kReadThreads / 64) + (threadIdx.x >> 6)] = acc;
}

}  // namespace

hipError_t launch_measure_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink,
                               hipStream_t stream) {
    const uint64_t n16 = bytes / 16;
    const uint64_t per = (n16 + (uint64_t)workgroups - 1) / (uint64_t)workgroups;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kReadThreads), 0, stream,
                       (const uint4*)buf, n16, per, sink);
    return hipGetLastError();
}

}  // namespace qkv
