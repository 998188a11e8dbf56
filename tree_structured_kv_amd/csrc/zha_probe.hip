// zha_probe.hip -- streaming HBM read probe (the achievable-bandwidth roof).
#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

__global__ __launch_bounds__(kBlock) void k_read_probe(const uint4 *buf, uint64_t n16, float *sink) {
    uint32_t acc = 0;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    uint64_t i = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        uint4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        uint4 a = buf[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    // keep the loads alive: a write that practically never happens
    if (acc == 0x9e3779b9u) atomicAdd(sink, 1.0f);
}

hipError_t launch_probe(const void *buf, uint64_t bytes, float *sink, hipStream_t st) {
    const uint64_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    const unsigned grid = 256 * 16;   // 16 workgroups per CU
    hipLaunchKernelGGL(k_read_probe, dim3(grid), dim3(kBlock), 0, st,
                       static_cast<const uint4 *>(buf), n16, sink);
    return hipGetLastError();
}

}  // namespace zha
