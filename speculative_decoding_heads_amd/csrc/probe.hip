// Streaming-read ceiling of the part: every workgroup reads its own contiguous
// share of a buffer with 16-byte loads, eight in flight per lane, and leaves one
// word per workgroup (so the loads cannot be dropped).  The achieved rate is the
// practical HBM read bandwidth the memory-bound kernels are compared with, next
// to the nominal 8 TB/s.
#include "common.h"
#include "medusa_model.h"

using namespace medusa;

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ src, size_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t acc = 0;
  size_t i = b0 + threadIdx.x;
  for (; i + (size_t)(kProbeUnroll - 1) * kProbeThreads < b1; i += (size_t)kProbeUnroll * kProbeThreads) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = src[i + (size_t)u * kProbeThreads];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < b1; i += kProbeThreads) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  __shared__ uint32_t s[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

}  // namespace

extern "C" int medusa_read_probe(const void* src, size_t bytes, int n_workgroups, uint32_t* sink,
                                 hipStream_t stream) {
  MEDUSA_REQUIRE(bytes >= 16 && bytes % 16 == 0 && n_workgroups >= 1, MEDUSA_ERR_ARG,
                 "read_probe: bytes must be a positive multiple of 16, workgroups >= 1");
  MEDUSA_REQUIRE(src && sink, MEDUSA_ERR_ARG, "read_probe: null pointer");
  MEDUSA_REQUIRE(((uintptr_t)src & 15) == 0, MEDUSA_ERR_ARG, "read_probe: source not 16-byte aligned");
  hipLaunchKernelGGL(read_probe_kernel, dim3(n_workgroups), dim3(kProbeThreads), 0, stream, (const uint4*)src,
                     bytes / 16, sink);
  return check_launch("read_probe");
}
