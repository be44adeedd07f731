// kernels.hpp — launch wrappers of the gfx950 kernels, called by the C ABI layer.
#pragma once

#include <hip/hip_ext.h>

#include "common.hpp"

namespace moe {

// Benchmark timer (moe_timer_start / moe_timer_read): hands out the next event
// pair when launches of kernel family `kid` are being timed.
bool timer_take(int kid, hipEvent_t* start, hipEvent_t* stop);

// Launch a kernel; when its family is being timed, launch it through
// hipExtLaunchKernelGGL so the events bracket exactly this kernel.
#define MOE_LAUNCH(KID, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                                    \
  do {                                                                                            \
    hipEvent_t moe_ev_a_, moe_ev_b_;                                                              \
    if (::moe::timer_take((KID), &moe_ev_a_, &moe_ev_b_))                                          \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, moe_ev_a_, moe_ev_b_, 0, __VA_ARGS__); \
    else                                                                                          \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);                         \
  } while (0)

constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;
constexpr int kMfmaLogitsMinT = 16;  // from this many tokens the router logits run on the matrix cores
constexpr int kMaxLogitSplits = 8;   // split-K partial planes of the batch router, at most
constexpr int kSplitRouterMinT = 128;  // from this many bf16 tokens the router runs on bf16 MFMA (split weights)
constexpr int kGroupLdsCells = 4096; // chunk x expert cells of the one-workgroup grouping (48 KiB of LDS); above, three kernels (measured faster from 8192 cells)


// Device buffers of the token-by-expert grouping.
struct GroupBufs {
  uint64_t* mask;    // [ceil(T/64)][E]
  int32_t* base;     // [ceil(T/64)][E]
  int32_t* counts;   // [E]
  int32_t* offsets;  // [E+1]
  int32_t* perm;     // [T*k]
  int32_t* uniq;     // [E]
  int32_t* n_uniq;   // [1]
};

// Experts as the kernels see them (byte pointers, decoded struct). E is the
// number of experts the routing ranges over. With a slot table (staged
// decode), expert e's weights sit at index slot_of[e] of a stack of `slots`
// experts; without one (slot_of null) at index e.
struct ExpertsDev {
  int E, H, I, scheme;
  const uint8_t* wgu;
  const uint16_t* sgu;
  const uint8_t* wd;
  const uint16_t* sd;
  const int32_t* slot_of = nullptr;
  int slots = 0;
};

// Index of expert e's weights: slot_of[e] when staged, else e. -1 for an
// expert without a slot in [0, slots): such an expert contributes nothing
// (kernels read index 0 with zero scales in its place).
__device__ __forceinline__ int expert_index(const ExpertsDev& ex, int e) {
  if (!ex.slot_of) return e;
  const int s = ex.slot_of[e];
  return s >= 0 && s < ex.slots ? s : -1;
}

// Split-K planes of the router logits the workspace holds room for: the batch
// router may write up to this many partial [T][E] planes (summed by the top-k).
inline int logits_max_splits(int64_t T, int64_t E) {
  if (T < kMfmaLogitsMinT) return 1;
  int64_t s = (1 << 20) / (T * E);
  return (int)(s < 1 ? 1 : s > kMaxLogitSplits ? kMaxLogitSplits : s);
}
// Writes *nsplit partial planes logits[s][T][E] (one for T < kMfmaLogitsMinT).
// split_ok: bf16 activations from kSplitRouterMinT tokens may take the
// split-weight bf16 kernel (otherwise the fp32 matrix-core kernel).
// ldr: row stride of R in elements (0: H).
hipError_t launch_logits(const void* x, int xtype, int T, int H, const float* R, int E, float* logits,
                         int* nsplit, bool split_ok, hipStream_t s, int64_t ldr = 0);
hipError_t launch_topk(const float* logits, int nsplit, int T, int E, int k, int renorm, int32_t* idx, float* gate,
                       int32_t* idx2, float* gate2, hipStream_t s);
hipError_t launch_group(const int32_t* idx, int T, int k, int E, const GroupBufs& g, hipStream_t s);

// Single-token decode: gate/up + SwiGLU into h[k][I] (fp16 for I <= 1024, where
// the one-wave-per-slot down kernel runs; fp32 otherwise), then down + combine.
// With logits != nullptr the routing is computed from them inside the gate/up
// kernel (and written to idx_ws/gate_ws and the optional user copies); otherwise
// idx/gate are read from idx_in/gate_in.
hipError_t launch_decode_t1(const void* x, int xtype, const ExpertsDev& ex, int k, int renorm,
                            const float* logits, const int32_t* idx_in, const float* gate_in,
                            int32_t* idx_ws, float* gate_ws, int32_t* idx_user, float* gate_user,
                            float* h, float* y, bool h32, hipStream_t s);

// Staged decode: copy experts[i] of pool into slot slots[i] of stack;
// out = slot_of[idx] for ids in [0, E), -1 for ids outside it.
hipError_t launch_stage_experts(const ExpertsDev& pool, const ExpertsDev& stack, const int32_t* experts,
                                const int32_t* slots, int n, hipStream_t s);
hipError_t launch_remap_ids(const int32_t* idx, int64_t n, const int32_t* slot_of, int E, int32_t* out,
                            hipStream_t s);

// Host replay of the expert-cache miss policies (arguments checked by the caller).
void miss_replay(const int32_t* idx, const float* gate, int T, int k, int E, int capacity, int policy,
                 float threshold, float beta, float* m, int32_t* sync, int32_t* bg, uint8_t* resident);

// Plain streaming read of `bytes` bytes (benchmark reference).
hipError_t launch_stream_read(const void* buf, int64_t bytes, hipStream_t s);

// Grouped decode for T > 1 (after launch_group): h[T*k][I], ys[T*k][H], y.
hipError_t launch_decode_grouped(const void* x, int xtype, int T, const ExpertsDev& ex, int k,
                                 const GroupBufs& g, const float* gate, float* h, float* ys, float* y,
                                 hipStream_t s);

// Gate-weighted combine (T > 1 paths): y[t] = sum over slots s, in order, of
// gate[t][s] * ys[t*k+s], per-slot rows fp32 (ys) or, when ys16 is non-null,
// fp16 rows times 2^ysig[t*k+s][m/32] (the grouped GEMM's).
hipError_t launch_combine(int T, int H, int k, const float* gate, const float* ys, const uint16_t* ys16,
                          const int32_t* ysig, float* y, hipStream_t s);

// Grouped MFMA GEMM path (after launch_group), for fp16 or bf16 activations:
// gate/up + SwiGLU into fp16 h [T*k][I] with one power-of-two exponent per tile
// in sig [T*k][ceil(I/64)], down into fp32 ys [T*k][H] (or y itself in
// per-slot mode), then the combine.
hipError_t launch_gemm_grouped(const void* x, int xtype, int T, const ExpertsDev& ex, int k, const GroupBufs& g,
                               const float* gate, uint16_t* h16, int32_t* sig, float* ys, float* y, hipStream_t s);

// Prerouter head weights as the kernels see them (fp32, the page's layout:
// w1 [F][H+2E], b1 [F] or null, w2 [E][F], b2 [E] or null, wl [E][H+2E]).
struct HeadDev {
  int H, E, F;
  const float* w1;
  const float* b1;
  const float* w2;
  const float* b2;
  const float* wl;
};
// fc1 + GELU into act [T][F] and the residual path + fc2's bias into part
// [T][E]; then part + fc2 into logits [T][E] and the router's top-k into
// idx/gate [T][k] (skipped when idx is null). cur/prev [T][k] or null. raw:
// scratch of head_raw_floats(T, E, F) floats (the matrix-core partial planes
// of a batch; unused below kMfmaLogitsMinT tokens).
inline int64_t head_raw_floats(int64_t T, int64_t E, int64_t F) {
  if (T < kMfmaLogitsMinT) return 0;
  return logits_max_splits(T, F) * T * F + logits_max_splits(T, E) * T * E;
}
hipError_t launch_prerouter(const void* x, int xtype, int T, const HeadDev& hd, const int32_t* cur,
                            const int32_t* prev, int k, int renorm, float* act, float* part, float* logits,
                            int32_t* idx, float* gate, float* raw, hipStream_t s);
// Quantized linear with an unmerged LoRA delta: u = A x into u [T][r] (when
// r > 0), then y [T][N] = W_q x + c * B u.
hipError_t launch_qlinear_lora(const void* x, int xtype, int T, int N, int K, int scheme, const uint8_t* codes,
                               const uint16_t* scales, const float* A, const float* B, int r, float c, float* u,
                               float* y, hipStream_t s);
// Prerouted decode of one token: experts on the predicted `logits` (top-k in
// the gate/up kernel, routing to idx_ws/gate_ws and the optional user copies),
// with the next layer's head run beside them: its logits for the next token go
// to logits_next. prev: this layer's routing at the previous token, or null.
// Valid when prerouted_t1_fusable() holds.
bool prerouted_t1_fusable(const ExpertsDev& ex, int xtype, const HeadDev& hd);
hipError_t launch_prerouted_t1(const void* x, int xtype, const ExpertsDev& ex, int k, int renorm,
                               const float* logits, int32_t* idx_ws, float* gate_ws, int32_t* idx_user,
                               float* gate_user, float* h, float* y, const HeadDev& hd, const int32_t* prev,
                               float* act, float* part, float* logits_next, hipStream_t s);
hipError_t launch_quantize(const float* w, int64_t rows, int K, int scheme, uint8_t* codes, uint16_t* scales,
                           hipStream_t s);

}  // namespace moe
