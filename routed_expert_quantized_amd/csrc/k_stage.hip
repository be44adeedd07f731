// k_stage.hip — expert staging for a resident stack of experts.
//
// "The Other Half of the Memory Wall: Serving 35B MoEs from SSD with Trained
// Routing Prediction" (xyznot.com), 重要用語 (glossary): in staged decode the
// expert indices are mapped through a slot table on the GPU into a fixed set of
// expert slots, so no memory is allocated per step; the incremental sticky-slot
// stack rewrites only the slots whose expert changed, in place. Here a stack is
// an ordinary expert pool (same H, I and codec) whose E is its slot count: an
// expert's gate/up codes, their scales, its down codes and their scales are four
// contiguous spans, copied into the spans of its slot.
#include <algorithm>

#include "kernels.hpp"

namespace moe {

// Grid: (chunk workgroups, n items). Item i copies the four spans of expert
// experts[i] of the pool into slot slots[i] of the stack, 16 bytes per thread
// per step; every span is a whole number of 16-byte pieces.
__global__ __launch_bounds__(256) void k_stage_experts(ExpertsDev pool, ExpertsDev stack,
                                                       const int32_t* __restrict__ experts,
                                                       const int32_t* __restrict__ slots) {
  const int e = experts[blockIdx.y], sl = slots[blockIdx.y];
  const int64_t H = pool.H, I = pool.I;
  const int64_t cb = pool.scheme == MOE_Q_SYM8 ? 1 : 2;  // codes per byte
  const int64_t span[4] = {2 * I * H / cb, 2 * I * (H / 32) * 2, H * I / cb, H * (I / 32) * 2};
  const uint8_t* src[4] = {pool.wgu, reinterpret_cast<const uint8_t*>(pool.sgu), pool.wd,
                           reinterpret_cast<const uint8_t*>(pool.sd)};
  uint8_t* dst[4] = {const_cast<uint8_t*>(stack.wgu), reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(stack.sgu)),
                     const_cast<uint8_t*>(stack.wd), reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(stack.sd))};
  const int64_t step = (int64_t)gridDim.x * 256;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const uint4* s = reinterpret_cast<const uint4*>(src[a] + (int64_t)e * span[a]);
    uint4* d = reinterpret_cast<uint4*>(dst[a] + (int64_t)sl * span[a]);
    const int64_t n16 = span[a] / 16;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += step) d[i] = s[i];
  }
}

__global__ __launch_bounds__(256) void k_remap_ids(const int32_t* __restrict__ idx, int64_t n,
                                                   const int32_t* __restrict__ slot_of, int E,
                                                   int32_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    const int e = idx[i];
    out[i] = e >= 0 && e < E ? slot_of[e] : -1;
  }
}

hipError_t launch_stage_experts(const ExpertsDev& pool, const ExpertsDev& stack, const int32_t* experts,
                                const int32_t* slots, int n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t biggest = 2LL * pool.I * pool.H / 16;  // 16-byte pieces of the largest span (sym8 gate/up)
  const unsigned chunks = (unsigned)std::min<int64_t>((biggest + 256 * 8 - 1) / (256 * 8), 512);
  hipLaunchKernelGGL(k_stage_experts, dim3(chunks, (unsigned)n), dim3(256), 0, s, pool, stack, experts, slots);
  return hipGetLastError();
}

hipError_t launch_remap_ids(const int32_t* idx, int64_t n, const int32_t* slot_of, int E, int32_t* out,
                            hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_remap_ids, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, idx, n, slot_of, E, out);
  return hipGetLastError();
}

}  // namespace moe
