// Streaming-read probe: the practical HBM read rate of a kernel that only
// reads, for a given number of workgroups (see moe_probe.h).
#include <hip/hip_runtime.h>

#include "moe_probe.h"

namespace moe {
moe_status set_error(moe_status code, const char* fmt, ...);
}

namespace {

constexpr int kThreads = 512;
constexpr int kUnroll = 4;   // 16-byte loads in flight per thread

__global__ __launch_bounds__(kThreads) void k_read_probe(const uint4* __restrict__ src, uint64_t n16,
                                                        uint32_t* __restrict__ sink) {
  // part of workgroup b: [b n16 / W, (b + 1) n16 / W) in 16-byte units, with
  // part boundaries on 1024-unit (16 KiB) multiples
  const uint64_t W = gridDim.x, blocks = n16 / 1024;
  const uint64_t p0 = (blockIdx.x * blocks / W) * 1024, p1 = ((blockIdx.x + 1) * blocks / W) * 1024;
  uint32_t acc = 0;
  for (uint64_t i = p0 + threadIdx.x; i < p1; i += kThreads * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t j = i + static_cast<uint64_t>(u) * kThreads;
      v[u] = j < p1 ? src[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // one word per workgroup: a fixed-order fold over the workgroup is not
  // needed (the value only keeps the loads alive), so lanes xor into LDS
  __shared__ uint32_t red;
  if (threadIdx.x == 0) red = 0;
  __syncthreads();
  atomicXor(&red, acc);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red;
}

}  // namespace

extern "C" moe_status moe_read_probe(const void* src, uint64_t bytes, int32_t n_workgroups, uint32_t* sink,
                                     moe_stream stream) {
  if (!src || !sink || (reinterpret_cast<uintptr_t>(src) & 255))
    return moe::set_error(MOE_EINVAL, "src (256-byte aligned) and sink are required");
  if (bytes == 0 || bytes % 16384) return moe::set_error(MOE_ESHAPE, "bytes=%llu must be a positive multiple of 16384",
                                                        (unsigned long long)bytes);
  if (n_workgroups < 1 || n_workgroups > 65536)
    return moe::set_error(MOE_ESHAPE, "n_workgroups=%d must be in [1, 65536]", n_workgroups);
  hipLaunchKernelGGL(k_read_probe, dim3(n_workgroups), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, sink);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return moe::set_error(MOE_EHIP, "read probe launch: %s", hipGetErrorString(e));
  return MOE_OK;
}
