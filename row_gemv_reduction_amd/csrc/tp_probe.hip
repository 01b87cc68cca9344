// Streaming-read ceiling of the device: a plain read of a buffer with
// 16-byte nontemporal loads, the access the decode kernels make of their
// weights ("Hosting Qwen on Blackwell", Decoders: a decode matmul costs what
// loading its weights costs). It does no arithmetic of the method; the
// benchmark times it over as many bytes as a decode step streams, so that
// the step's bandwidth can be set against what a read alone achieves on the
// same device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tp_device.h"
#include "tp_internal.h"

namespace {

using namespace tpdev;

constexpr int kProbeBlock = 512;
constexpr int kProbeUnroll = 16;

// Grid-stride over 16-byte vectors; each lane keeps kProbeUnroll loads in
// flight. The vectors are folded with XOR into one word per workgroup,
// stored to `sink`, so no load can be dropped.
__global__ __launch_bounds__(kProbeBlock) void stream_read_kernel(const u32x4_t* __restrict__ p,
                                                                  int64_t n16, uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * kProbeBlock;
    int64_t i = (int64_t)blockIdx.x * kProbeBlock + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        u32x4_t v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4_t v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    acc ^= __shfl_xor(acc, 1);
    acc ^= __shfl_xor(acc, 2);
    acc ^= __shfl_xor(acc, 4);
    acc ^= __shfl_xor(acc, 8);
    acc ^= __shfl_xor(acc, 16);
    acc ^= __shfl_xor(acc, 32);
    __shared__ uint32_t part[kProbeBlock / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int w = 0; w < kProbeBlock / 64; ++w) s ^= part[w];
        sink[blockIdx.x] = s;
    }
}

}  // namespace

extern "C" tp_status tp_stream_read_probe(const void* buf, int64_t bytes, uint32_t* sink,
                                          int32_t workgroups, void* stream) {
    if (!buf || !sink || bytes < 0 || workgroups < 1 || workgroups > 65536) return TP_ERR_INVALID_ARG;
    if (((uintptr_t)buf & 15) || ((uintptr_t)sink & 15) || (bytes & 15)) return TP_ERR_ALIGNMENT;
    if (bytes == 0) return TP_OK;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kProbeBlock), 0,
                       (hipStream_t)stream, static_cast<const u32x4_t*>(buf), bytes / 16, sink);
    return tp_launch_status(stream);
}
