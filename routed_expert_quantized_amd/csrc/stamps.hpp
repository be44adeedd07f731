// stamps.hpp — opt-in per-workgroup timestamps for the single-token chain
// (router row kernel, gate/up, down).
//
// Only a build with -DMOE_STAMPS (libmoe_stamps.so, made by
// `python -m routed_expert_quantized_amd.build --stamps`) records anything;
// in every other build the macros below expand to nothing and the kernels are
// unchanged. A stamp is the GPU's constant-rate real-time counter
// (s_memrealtime), stored by thread 0 of a workgroup whose index is below
// kStampCols into a table of its translation unit; extern "C" readers copy a
// table to the host
// (moe_stamps_read_route, moe_stamps_read_decode, and moe_stamps_clock_khz
// for the counter's frequency; exported by that build only, so they are not in
// the public header).
//
// MOE_STAMP_LANDED first waits, in wave 0, for every load that wave has in
// flight, so it changes that wave's schedule: a timestamp build gives a
// timeline of the chain, not kernel times.
//
// The grouped GEMM uses the same build differently: each wave sums the shader
// clock (s_memtime, read between scheduling barriers so that no instruction
// moves across a reading) spent in each phase of its tiles, and adds the sums
// into a small table per kernel mode (moe_stamps_read_gemm,
// moe_stamps_zero_gemm). MOE_STAMPS_ONLY(...) keeps its argument only in this
// build.
#pragma once

namespace moe {
constexpr int kStampCols = 1024;
}

#ifdef MOE_STAMPS
#define MOE_STAMP_TABLE(name, rows) __device__ unsigned long long name[rows][::moe::kStampCols]
#define MOE_STAMP(table, row, bid)                                                 \
  do {                                                                             \
    if (threadIdx.x == 0 && (int)(bid) < ::moe::kStampCols)                       \
      table[row][(int)(bid)] = __builtin_amdgcn_s_memrealtime();                   \
  } while (0)
#define MOE_STAMP_LANDED(table, row, bid)                                          \
  do {                                                                             \
    __builtin_amdgcn_sched_barrier(0);                                             \
    if (threadIdx.x < 64) {                                                        \
      __builtin_amdgcn_s_waitcnt(0);                                               \
      MOE_STAMP(table, row, bid);                                                  \
    }                                                                              \
    __builtin_amdgcn_sched_barrier(0);                                             \
  } while (0)
#define MOE_STAMP_READER(fn, table)                                                \
  extern "C" int fn(void* host) {                                                  \
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(table), sizeof(table));       \
  }
#define MOE_STAMPS_ONLY(...) __VA_ARGS__
namespace moe {
__device__ __forceinline__ unsigned long long stamp_clock() {
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t = __builtin_amdgcn_s_memtime();
  __builtin_amdgcn_sched_barrier(0);
  return t;
}
}  // namespace moe
#else
#define MOE_STAMP_TABLE(name, rows) static_assert(true, "")
#define MOE_STAMP(table, row, bid) \
  do {                             \
  } while (0)
#define MOE_STAMP_LANDED(table, row, bid) \
  do {                                    \
  } while (0)
#define MOE_STAMP_READER(fn, table) static_assert(true, "")
#define MOE_STAMPS_ONLY(...)
#endif
