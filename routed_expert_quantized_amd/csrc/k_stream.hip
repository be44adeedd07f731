// k_stream.hip — a plain streaming read, the reference for achievable HBM
// bandwidth at a given transfer size (benchmark support, not part of the layer).
#include "kernels.hpp"

namespace moe {

// Each thread issues kStreamLoads coalesced 16-byte loads (thread-contiguous
// within each load round) before using any of them; the values only feed a
// store the host disables (sink == nullptr), which keeps the loads alive.
constexpr int kStreamLoads = 4;

__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ p, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nt = (int64_t)gridDim.x * blockDim.x;
  u32x4 v[kStreamLoads];
#pragma unroll
  for (int i = 0; i < kStreamLoads; ++i) {
    const int64_t j = i * nt + gid;
    v[i] = j < n16 ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t a = 0;
#pragma unroll
  for (int i = 0; i < kStreamLoads; ++i) a ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (sink) sink[gid] = a;
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t per_wg = 256 * kStreamLoads;
  const dim3 grid((unsigned)((n16 + per_wg - 1) / per_wg));
  hipLaunchKernelGGL(k_stream_read, grid, dim3(256), 0, s, reinterpret_cast<const u32x4*>(buf), n16,
                     static_cast<uint32_t*>(nullptr));
  return hipGetLastError();
}

}  // namespace moe
