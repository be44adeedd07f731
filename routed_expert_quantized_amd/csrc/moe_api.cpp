// moe_api.cpp — host side of the C ABI declared in include/moe.h: argument
// checks, workspace layout and kernel dispatch. No allocation, no host sync.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "moe.h"

// Scratch of moe_layer_forward_noalloc: a file-scope device array, one copy per
// GPU. In host code its name stands for the host-side shadow, not a device
// address, so kernels and copies only ever get the address looked up by
// scratch_address() below.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status ok() {
  g_err.clear();
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Scratch regions inside the caller's workspace, each 256-byte aligned.
struct Layout {
  size_t logits, idx, gate, mask, base, counts, offsets, perm, uniq, n_uniq, h, hsig, ys, total;
};

Layout layout(int64_t T, int64_t E, int64_t H, int64_t I, int64_t k) {
  Layout L{};
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    const size_t o = off;
    off += ((size_t)bytes + 255) & ~(size_t)255;
    return o;
  };
  const int64_t C = (T + 63) / 64;
  L.logits = take(T * E * 4 * moe::logits_max_splits(T, E));
  L.idx = take(T * k * 4);
  L.gate = take(T * k * 4);
  L.mask = take(C * E * 8);
  L.base = take(C * E * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.perm = take(T * k * 4);
  L.uniq = take(E * 4);
  L.n_uniq = take(4);
  L.h = take(T * k * I * 4);
  L.hsig = take(T * k * ((I + 63) / 64) * 4);  // the grouped GEMM's tile exponents of h
  L.ys = take(T * k * H * 4);
  L.total = off;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

moe::GroupBufs group_bufs(void* ws, const Layout& L) {
  return moe::GroupBufs{at<uint64_t>(ws, L.mask), at<int32_t>(ws, L.base), at<int32_t>(ws, L.counts),
                        at<int32_t>(ws, L.offsets), at<int32_t>(ws, L.perm), at<int32_t>(ws, L.uniq),
                        at<int32_t>(ws, L.n_uniq)};
}

bool shape_ok(int64_t T, int64_t E, int64_t H, int64_t I, int64_t k) {
  return T >= 1 && T <= 65536 && E >= 1 && E <= moe::kMaxE && H >= 32 && H <= 4096 && H % 32 == 0 &&
         I >= 32 && I <= 4096 && I % 32 == 0 && k >= 1 && k <= std::min<int64_t>(E, moe::kMaxK);
}

moe_status check_shape(int64_t T, int64_t E, int64_t H, int64_t I, int64_t k) {
  if (T < 1 || T > 65536) return fail(MOE_ERR_INVALID_ARG, "T=%lld outside [1, 65536]", (long long)T);
  if (E < 1 || E > moe::kMaxE) return fail(MOE_ERR_INVALID_ARG, "E=%lld outside [1, %d]", (long long)E, moe::kMaxE);
  if (H < 32 || H > 4096 || H % 32)
    return fail(MOE_ERR_INVALID_ARG, "H=%lld must be a multiple of 32 in [32, 4096]", (long long)H);
  if (I < 32 || I > 4096 || I % 32)
    return fail(MOE_ERR_INVALID_ARG, "I=%lld must be a multiple of 32 in [32, 4096]", (long long)I);
  if (k < 1 || k > std::min<int64_t>(E, moe::kMaxK))
    return fail(MOE_ERR_INVALID_ARG, "k=%lld outside [1, min(E, %d)]", (long long)k, moe::kMaxK);
  return MOE_OK;
}

// The expert-path flags: at most one path, and the grouped GEMM only for
// 16-bit activations (its MFMA operands are the activations as given).
moe_status check_path_flags(uint32_t flags, int32_t xtype) {
  if ((flags & MOE_FLAG_PATH_GATHER) && (flags & MOE_FLAG_PATH_GEMM))
    return fail(MOE_ERR_INVALID_ARG, "both path flags are set");
  if (flags & ~(uint32_t)(MOE_FLAG_RENORM | MOE_FLAG_PATH_GATHER | MOE_FLAG_PATH_GEMM | MOE_FLAG_H_FP32))
    return fail(MOE_ERR_UNSUPPORTED, "unknown flag bits 0x%x", flags);
  if ((flags & MOE_FLAG_PATH_GEMM) && xtype == MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "the grouped GEMM path takes fp16 or bf16 activations, not fp32");
  return MOE_OK;
}

moe_status check_ws(void* ws, size_t ws_bytes, const Layout& L) {
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace pointer is NULL");
  if (!aligned(ws, 256)) return fail(MOE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, L.total);
  return MOE_OK;
}

moe_status check_x(const void* x, int32_t xtype) {
  if (!x) return fail(MOE_ERR_INVALID_ARG, "x is NULL");
  if (xtype < MOE_F32 || xtype > MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "unknown activation type %d", xtype);
  if (!aligned(x, 16)) return fail(MOE_ERR_INVALID_ARG, "x is not 16-byte aligned");
  return MOE_OK;
}

moe_status check_experts(const moe_experts* ex, moe::ExpertsDev* d) {
  if (!ex) return fail(MOE_ERR_INVALID_ARG, "experts struct is NULL");
  if (ex->scheme != MOE_Q_SYM8 && ex->scheme != MOE_Q_INT4)
    return fail(MOE_ERR_UNSUPPORTED, "unknown weight codec %d", ex->scheme);
  if (!ex->w_gate_up || !ex->s_gate_up || !ex->w_down || !ex->s_down)
    return fail(MOE_ERR_INVALID_ARG, "an expert weight or scale pointer is NULL");
  if (!aligned(ex->w_gate_up, 16) || !aligned(ex->w_down, 16) || !aligned(ex->s_gate_up, 2) ||
      !aligned(ex->s_down, 2))
    return fail(MOE_ERR_INVALID_ARG, "expert codes must be 16-byte aligned and scales 2-byte aligned");
  *d = moe::ExpertsDev{ex->E, ex->H, ex->I, ex->scheme, static_cast<const uint8_t*>(ex->w_gate_up), ex->s_gate_up,
                       static_cast<const uint8_t*>(ex->w_down), ex->s_down};
  return MOE_OK;
}

// Expert stage shared by moe_gather_qmm_forward and moe_layer_forward.
moe_status run_experts(const void* x, int32_t xtype, int32_t T, const moe::ExpertsDev& d, int32_t k,
                       const int32_t* idx, const float* gate, float* y, uint32_t flags, void* ws,
                       const Layout& L, hipStream_t s) {
  float* h = at<float>(ws, L.h);
  // Path choice: the grouped MFMA GEMM when asked, and by default for T > 1
  // with 16-bit activations; the gathered matvec for a single token, for fp32
  // activations or when asked (validation has rejected the GEMM with fp32).
  const bool gemm = (flags & MOE_FLAG_PATH_GEMM) || (!(flags & MOE_FLAG_PATH_GATHER) && T > 1 && xtype != MOE_F32);
  if (T == 1 && !gemm)
    return hip_status(moe::launch_decode_t1(x, xtype, d, k, 0, nullptr, idx, gate, nullptr, nullptr, nullptr,
                                            nullptr, h, y, (flags & MOE_FLAG_H_FP32) != 0, s),
                      "decode (one token)");
  const moe::GroupBufs g = group_bufs(ws, L);
  hipError_t e = moe::launch_group(idx, T, k, d.E, g, s);
  if (e != hipSuccess) return hip_status(e, "grouping");
  if (gemm)
    return hip_status(moe::launch_gemm_grouped(x, xtype, T, d, k, g, gate, reinterpret_cast<uint16_t*>(h),
                                               at<int32_t>(ws, L.hsig), at<float>(ws, L.ys), y, s),
                      "grouped GEMM");
  return hip_status(moe::launch_decode_grouped(x, xtype, T, d, k, g, gate, h, at<float>(ws, L.ys), y, s),
                    "decode (grouped)");
}

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_dev[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch array: hipGetSymbolAddress once per
// device, with that device current, then the cached pointer.
moe_status scratch_address(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  if (s) {
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(s, &sd);
    if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
    if (sd != dev) return fail(MOE_ERR_INVALID_ARG, "stream belongs to device %d, the current device is %d", sd, dev);
  }
  void* p = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_dev[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
      if (!p || !aligned(p, 256)) return fail(MOE_ERR_HIP, "scratch address %p is not 256-byte aligned", p);
      g_scratch_dev[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

// Benchmark timer state (see moe_timer_start).
struct KernelTimer {
  int kid = -1;
  int cap = 0;
  int used = 0;
  std::vector<hipEvent_t> start, stop;
};
KernelTimer g_timer;

}  // namespace

namespace moe {
bool timer_take(int kid, hipEvent_t* start, hipEvent_t* stop) {
  if (g_timer.kid != kid || g_timer.used >= g_timer.cap) return false;
  *start = g_timer.start[g_timer.used];
  *stop = g_timer.stop[g_timer.used];
  ++g_timer.used;
  return true;
}
}  // namespace moe

namespace {
// The expert layer after the router's gate linear: top-k on `logits` ([nsplit]
// partial planes of [T][E]), then the routed experts.
moe_status layer_from_logits(const void* x, int32_t xtype, int32_t T, const moe::ExpertsDev& d, int32_t k,
                             uint32_t flags, const float* logits, int nsplit, float* y, int32_t* topk_idx_out,
                             float* topk_gate_out, void* ws, const Layout& L, hipStream_t s) {
  const int renorm = (flags & MOE_FLAG_RENORM) ? 1 : 0;
  int32_t* idx = at<int32_t>(ws, L.idx);
  float* gate = at<float>(ws, L.gate);
  if (T == 1 && !(flags & MOE_FLAG_PATH_GEMM))
    return hip_status(moe::launch_decode_t1(x, xtype, d, k, renorm, logits, nullptr, nullptr, idx, gate,
                                            topk_idx_out, topk_gate_out, at<float>(ws, L.h), y,
                                            (flags & MOE_FLAG_H_FP32) != 0, s),
                      "decode (one token)");
  hipError_t e = moe::launch_topk(logits, nsplit, T, d.E, k, renorm, idx, gate, topk_idx_out, topk_gate_out, s);
  if (e != hipSuccess) return hip_status(e, "top-k");
  return run_experts(x, xtype, T, d, k, idx, gate, y, flags, ws, L, s);
}

// Checks of a layer call other than its workspace; fills the decoded experts
// and the workspace layout.
moe_status check_layer_shapes(const void* x, int32_t xtype, int32_t T, const moe_experts* ex, int32_t k,
                              uint32_t flags, const float* y, moe::ExpertsDev* d, Layout* L) {
  moe_status st;
  if ((st = check_x(x, xtype))) return st;
  if ((st = check_experts(ex, d))) return st;
  if ((st = check_shape(T, d->E, d->H, d->I, k))) return st;
  if (!y) return fail(MOE_ERR_INVALID_ARG, "y is NULL");
  if (!aligned(y, 16)) return fail(MOE_ERR_INVALID_ARG, "y is not 16-byte aligned");
  if ((st = check_path_flags(flags, xtype))) return st;
  *L = layout(T, d->E, d->H, d->I, k);
  return MOE_OK;
}

moe_status check_layer_args(const void* x, int32_t xtype, int32_t T, const moe_experts* ex, int32_t k, uint32_t flags,
                            const float* y, void* ws, size_t ws_bytes, moe::ExpertsDev* d, Layout* L) {
  moe_status st;
  if ((st = check_layer_shapes(x, xtype, T, ex, k, flags, y, d, L))) return st;
  return check_ws(ws, ws_bytes, *L);
}

moe_status check_router(const float* router_w) {
  if (!router_w) return fail(MOE_ERR_INVALID_ARG, "router_w is NULL");
  if (!aligned(router_w, 16)) return fail(MOE_ERR_INVALID_ARG, "router_w is not 16-byte aligned");
  return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_timer_start(int32_t kernel, int32_t capacity) {
  if (kernel < 0 || kernel >= MOE_KERNEL_COUNT) return fail(MOE_ERR_INVALID_ARG, "unknown kernel id %d", kernel);
  if (capacity < 1 || capacity > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "capacity %d outside [1, 2^20]", capacity);
  while ((int)g_timer.start.size() < capacity) {
    hipEvent_t a, b;
    hipError_t e = hipEventCreate(&a);
    if (e == hipSuccess) e = hipEventCreate(&b);
    if (e != hipSuccess) return hip_status(e, "timer events");
    g_timer.start.push_back(a);
    g_timer.stop.push_back(b);
  }
  g_timer.kid = kernel;
  g_timer.cap = capacity;
  g_timer.used = 0;
  return ok();
}

moe_status moe_timer_read(float* ms, int32_t capacity, int32_t* count) {
  if (!ms || !count) return fail(MOE_ERR_INVALID_ARG, "ms or count is NULL");
  const int n = std::min(g_timer.used, (int)capacity);
  for (int i = 0; i < n; ++i) {
    hipError_t e = hipEventSynchronize(g_timer.stop[i]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms[i], g_timer.start[i], g_timer.stop[i]);
    if (e != hipSuccess) return hip_status(e, "timer read");
  }
  *count = n;
  g_timer.kid = -1;
  g_timer.used = 0;
  return ok();
}

size_t moe_workspace_bytes(int32_t T, int32_t E, int32_t H, int32_t I, int32_t k, int32_t scheme) {
  if (!shape_ok(T, E, H, I, k) || (scheme != MOE_Q_SYM8 && scheme != MOE_Q_INT4)) return 0;
  return layout(T, E, H, I, k).total;
}

moe_status moe_route(const void* x, int32_t xtype, int32_t T, int32_t H, const float* router_w, int32_t E,
                     int32_t k, uint32_t flags, int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes,
                     void* stream) {
  moe_status st;
  if ((st = check_x(x, xtype))) return st;
  if ((st = check_shape(T, E, H, 32, k))) return st;
  if (!router_w || !topk_idx || !topk_gate) return fail(MOE_ERR_INVALID_ARG, "router_w, topk_idx or topk_gate is NULL");
  if (!aligned(router_w, 16)) return fail(MOE_ERR_INVALID_ARG, "router_w is not 16-byte aligned");
  if (flags & ~(uint32_t)(MOE_FLAG_RENORM | MOE_FLAG_PATH_GATHER | MOE_FLAG_PATH_GEMM))
    return fail(MOE_ERR_UNSUPPORTED, "unknown flag bits 0x%x", flags);
  const Layout L = layout(T, E, H, 32, k);
  if ((st = check_ws(ws, ws_bytes, L))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* logits = at<float>(ws, L.logits);
  int nsplit = 1;
  hipError_t e = moe::launch_logits(x, xtype, T, H, router_w, E, logits, &nsplit,
                                    true, s);
  if (e != hipSuccess) return hip_status(e, "router logits");
  return hip_status(moe::launch_topk(logits, nsplit, T, E, k, (flags & MOE_FLAG_RENORM) ? 1 : 0, topk_idx, topk_gate,
                                     nullptr, nullptr, s),
                    "top-k");
}

moe_status moe_group(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, int32_t* counts, int32_t* offsets,
                     int32_t* perm, int32_t* uniq, int32_t* n_uniq, void* ws, size_t ws_bytes, void* stream) {
  moe_status st;
  if ((st = check_shape(T, E, 32, 32, k))) return st;
  if (!topk_idx || !counts || !offsets || !perm || !uniq || !n_uniq)
    return fail(MOE_ERR_INVALID_ARG, "a grouping pointer is NULL");
  const Layout L = layout(T, E, 32, 32, k);
  if ((st = check_ws(ws, ws_bytes, L))) return st;
  moe::GroupBufs g = group_bufs(ws, L);
  g.counts = counts;
  g.offsets = offsets;
  g.perm = perm;
  g.uniq = uniq;
  g.n_uniq = n_uniq;
  return hip_status(moe::launch_group(topk_idx, T, k, E, g, static_cast<hipStream_t>(stream)), "grouping");
}

moe_status moe_gather_qmm_forward(const void* x, int32_t xtype, int32_t T, const moe_experts* ex, int32_t k,
                                  const int32_t* topk_idx, const float* topk_gate, float* y, uint32_t flags,
                                  void* ws, size_t ws_bytes, void* stream) {
  moe_status st;
  moe::ExpertsDev d;
  if ((st = check_x(x, xtype))) return st;
  if ((st = check_experts(ex, &d))) return st;
  if ((st = check_shape(T, d.E, d.H, d.I, k))) return st;
  if (!topk_idx || !y) return fail(MOE_ERR_INVALID_ARG, "topk_idx or y is NULL");
  if (!aligned(y, 16)) return fail(MOE_ERR_INVALID_ARG, "y is not 16-byte aligned");
  if ((st = check_path_flags(flags, xtype))) return st;
  const Layout L = layout(T, d.E, d.H, d.I, k);
  if ((st = check_ws(ws, ws_bytes, L))) return st;
  return run_experts(x, xtype, T, d, k, topk_idx, topk_gate, y, flags, ws, L, static_cast<hipStream_t>(stream));
}

moe_status moe_layer_forward(const void* x, int32_t xtype, int32_t T, const float* router_w, const moe_experts* ex,
                             int32_t k, uint32_t flags, float* y, int32_t* topk_idx_out, float* topk_gate_out,
                             void* ws, size_t ws_bytes, void* stream) {
  moe_status st;
  moe::ExpertsDev d;
  Layout L;
  if ((st = check_layer_args(x, xtype, T, ex, k, flags, y, ws, ws_bytes, &d, &L))) return st;
  if ((st = check_router(router_w))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* logits = at<float>(ws, L.logits);
  int nsplit = 1;
  hipError_t e = moe::launch_logits(x, xtype, T, d.H, router_w, d.E, logits, &nsplit,
                                    true, s);
  if (e != hipSuccess) return hip_status(e, "router logits");
  return layer_from_logits(x, xtype, T, d, k, flags, logits, nsplit, y, topk_idx_out, topk_gate_out, ws, L, s);
}

moe_status moe_layer_forward_staged(const void* x, int32_t xtype, int32_t T, const float* router_w, int32_t E,
                                    const moe_experts* stack, const int32_t* slot_of, int32_t k, uint32_t flags,
                                    float* y, int32_t* topk_idx_out, float* topk_gate_out, void* ws,
                                    size_t ws_bytes, void* stream) {
  moe_status st;
  moe::ExpertsDev d;
  Layout L;
  if (!stack) return fail(MOE_ERR_INVALID_ARG, "stack struct is NULL");
  if (stack->E < 1 || stack->E > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "stack slots %d outside [1, 2^20]", stack->E);
  if (!slot_of) return fail(MOE_ERR_INVALID_ARG, "slot_of is NULL");
  if (!aligned(slot_of, 4)) return fail(MOE_ERR_INVALID_ARG, "slot_of is not 4-byte aligned");
  // the routing ranges over E experts; the weights sit in the stack's slots
  moe_experts routed = *stack;
  routed.E = E;
  if ((st = check_layer_args(x, xtype, T, &routed, k, flags, y, ws, ws_bytes, &d, &L))) return st;
  if ((st = check_router(router_w))) return st;
  d.slot_of = slot_of;
  d.slots = stack->E;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* logits = at<float>(ws, L.logits);
  int nsplit = 1;
  hipError_t e = moe::launch_logits(x, xtype, T, d.H, router_w, d.E, logits, &nsplit,
                                    true, s);
  if (e != hipSuccess) return hip_status(e, "router logits");
  return layer_from_logits(x, xtype, T, d, k, flags, logits, nsplit, y, topk_idx_out, topk_gate_out, ws, L, s);
}

moe_status moe_layer_forward_noalloc(const void* x, int32_t xtype, int32_t T, const float* router_w,
                                     const moe_experts* ex, int32_t k, uint32_t flags, float* y,
                                     int32_t* topk_idx_out, float* topk_gate_out, void* stream) {
  moe_status st;
  moe::ExpertsDev d;
  Layout L;
  // every check of moe_layer_forward, with the scratch size in place of the
  // workspace's, before anything touches the device
  if ((st = check_layer_shapes(x, xtype, T, ex, k, flags, y, &d, &L))) return st;
  if ((st = check_router(router_w))) return st;
  if (L.total > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE, "these sizes need %zu bytes of scratch; the static scratch holds %zu", L.total,
                (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((st = scratch_address(s, &ws))) return st;
  return moe_layer_forward(x, xtype, T, router_w, ex, k, flags, y, topk_idx_out, topk_gate_out, ws,
                           MOE_NOALLOC_SCRATCH_BYTES, stream);
}

moe_status moe_experts_from_logits(const void* x, int32_t xtype, int32_t T, const float* logits,
                                   const moe_experts* ex, int32_t k, uint32_t flags, float* y, int32_t* topk_idx_out,
                                   float* topk_gate_out, void* ws, size_t ws_bytes, void* stream) {
  moe_status st;
  moe::ExpertsDev d;
  Layout L;
  if ((st = check_layer_args(x, xtype, T, ex, k, flags, y, ws, ws_bytes, &d, &L))) return st;
  if (!logits) return fail(MOE_ERR_INVALID_ARG, "logits is NULL");
  if (!aligned(logits, 16)) return fail(MOE_ERR_INVALID_ARG, "logits is not 16-byte aligned");
  return layer_from_logits(x, xtype, T, d, k, flags, logits, 1, y, topk_idx_out, topk_gate_out, ws, L,
                           static_cast<hipStream_t>(stream));
}

moe_status moe_quantize(const float* w, int64_t rows, int32_t K, int32_t scheme, void* codes, uint16_t* scales,
                        void* stream) {
  if (!w || !codes || !scales) return fail(MOE_ERR_INVALID_ARG, "w, codes or scales is NULL");
  if (rows < 0 || K <= 0 || K % 32) return fail(MOE_ERR_INVALID_ARG, "rows=%lld, K=%d: K must be a positive multiple of 32", (long long)rows, K);
  if (scheme != MOE_Q_SYM8 && scheme != MOE_Q_INT4) return fail(MOE_ERR_UNSUPPORTED, "unknown weight codec %d", scheme);
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 2))
    return fail(MOE_ERR_INVALID_ARG, "w and codes must be 16-byte aligned, scales 2-byte aligned");
  return hip_status(moe::launch_quantize(w, rows, K, scheme, static_cast<uint8_t*>(codes), scales,
                                         static_cast<hipStream_t>(stream)),
                    "quantize");
}

moe_status moe_miss_replay(const int32_t* topk_idx, const float* topk_gate, int32_t T, int32_t k, int32_t E,
                           int32_t capacity, int32_t policy, float threshold, float admit_beta, float* m,
                           int32_t* sync_fetches, int32_t* bg_fetches, uint8_t* resident) {
  if (!topk_idx || !topk_gate || !m || !sync_fetches || !bg_fetches)
    return fail(MOE_ERR_INVALID_ARG, "topk_idx, topk_gate, m, sync_fetches or bg_fetches is NULL");
  if (T < 0 || k < 1 || capacity < k || E < capacity || E > (1 << 20))
    return fail(MOE_ERR_INVALID_ARG, "T=%d k=%d capacity=%d E=%d: need T >= 0 and 1 <= k <= capacity <= E <= 2^20",
                T, k, capacity, E);
  if (policy != MOE_MISS_FETCH_ALL && policy != MOE_MISS_RULE && policy != MOE_MISS_FIRST_CHOICE)
    return fail(MOE_ERR_UNSUPPORTED, "unknown miss policy %d", policy);
  for (int64_t t = 0; t < T; ++t)
    for (int s = 0; s < k; ++s) {
      const int32_t e = topk_idx[t * k + s];
      if (e < 0 || e >= E) return fail(MOE_ERR_INVALID_ARG, "token %lld slot %d: expert %d out of [0, %d)", (long long)t, s, e, E);
      for (int j = 0; j < s; ++j)
        if (topk_idx[t * k + j] == e) return fail(MOE_ERR_INVALID_ARG, "token %lld: expert %d selected twice", (long long)t, e);
    }
  moe::miss_replay(topk_idx, topk_gate, T, k, E, capacity, policy, threshold, admit_beta, m, sync_fetches, bg_fetches,
                   resident);
  return ok();
}

moe_status moe_stage_experts(const moe_experts* pool, const moe_experts* stack, const int32_t* experts,
                             const int32_t* slots, int32_t n, void* stream) {
  moe_status st;
  moe::ExpertsDev p, q;
  if ((st = check_experts(pool, &p))) return st;
  if ((st = check_experts(stack, &q))) return st;
  if (p.H != q.H || p.I != q.I || p.scheme != q.scheme)
    return fail(MOE_ERR_INVALID_ARG, "stack (H=%d, I=%d, codec %d) differs from the pool (H=%d, I=%d, codec %d)",
                q.H, q.I, q.scheme, p.H, p.I, p.scheme);
  if ((st = check_shape(1, p.E, p.H, p.I, 1))) return st;
  if (q.E < 1 || q.E > p.E) return fail(MOE_ERR_INVALID_ARG, "stack slots E=%d outside [1, %d]", q.E, p.E);
  if (!aligned(pool->s_gate_up, 16) || !aligned(pool->s_down, 16) || !aligned(stack->s_gate_up, 16) ||
      !aligned(stack->s_down, 16))
    return fail(MOE_ERR_INVALID_ARG, "scales must be 16-byte aligned for staging");
  if (n < 0 || (n > 0 && (!experts || !slots))) return fail(MOE_ERR_INVALID_ARG, "n=%d, experts or slots NULL", n);
  return hip_status(moe::launch_stage_experts(p, q, experts, slots, n, static_cast<hipStream_t>(stream)),
                    "stage experts");
}

moe_status moe_remap_ids(const int32_t* idx, int64_t n, const int32_t* slot_of, int32_t E, int32_t* out,
                         void* stream) {
  if (n < 0 || E < 1) return fail(MOE_ERR_INVALID_ARG, "n=%lld E=%d", (long long)n, E);
  if (n > 0 && (!idx || !slot_of || !out)) return fail(MOE_ERR_INVALID_ARG, "idx, slot_of or out is NULL");
  return hip_status(moe::launch_remap_ids(idx, n, slot_of, E, out, static_cast<hipStream_t>(stream)), "remap ids");
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static bool head_shape_ok(int64_t T, int64_t E, int64_t F) {
  return T >= 1 && T <= 65536 && E >= 2 && E <= moe::kMaxE && E % 2 == 0 && F >= 32 && F <= 4096 && F % 32 == 0;
}

static moe_status check_head(const moe_prerouter* head, int64_t T, int64_t k) {
  moe_status st;
  if (!head) return fail(MOE_ERR_INVALID_ARG, "prerouter struct is NULL");
  const int64_t H = head->H, E = head->E, F = head->F;
  if ((st = check_shape(T, E, H, 32, k))) return st;
  if (E < 2 || E % 2) return fail(MOE_ERR_INVALID_ARG, "E=%lld must be even and >= 2 for the prerouter", (long long)E);
  if (F < 32 || F > 4096 || F % 32)
    return fail(MOE_ERR_INVALID_ARG, "F=%lld must be a multiple of 32 in [32, 4096]", (long long)F);
  if (!head->w1 || !head->w2 || !head->wl) return fail(MOE_ERR_INVALID_ARG, "w1, w2 or wl is NULL");
  if (!aligned(head->w1, 16) || !aligned(head->w2, 16) || !aligned(head->wl, 16) ||
      (head->b1 && !aligned(head->b1, 4)) || (head->b2 && !aligned(head->b2, 4)))
    return fail(MOE_ERR_INVALID_ARG, "head weights must be 16-byte aligned and biases 4-byte aligned");
  return MOE_OK;
}

size_t moe_prerouter_workspace_bytes(int32_t T, int32_t E, int32_t F) {
  if (!head_shape_ok(T, E, F)) return 0;
  // fc1 activations [T][F], residual-path partials [T][E], logits [T][E], and
  // for a batch the matrix-core partial planes
  return align256((size_t)T * F * 4) + 2 * align256((size_t)T * E * 4) +
         align256((size_t)moe::head_raw_floats(T, E, F) * 4);
}

moe_status moe_prerouter_forward(const void* x, int32_t xtype, int32_t T, const moe_prerouter* head,
                                 const int32_t* cur, const int32_t* prev, int32_t k, uint32_t flags,
                                 int32_t* topk_idx, float* topk_gate, float* logits, void* ws, size_t ws_bytes,
                                 void* stream) {
  moe_status st;
  if ((st = check_x(x, xtype))) return st;
  if ((st = check_head(head, T, k))) return st;
  const int64_t H = head->H, E = head->E, F = head->F;
  if ((cur && !aligned(cur, 4)) || (prev && !aligned(prev, 4)))
    return fail(MOE_ERR_INVALID_ARG, "cur or prev is not 4-byte aligned");
  if (!topk_idx != !topk_gate) return fail(MOE_ERR_INVALID_ARG, "only one of topk_idx and topk_gate is NULL");
  if (!topk_idx && !logits) return fail(MOE_ERR_INVALID_ARG, "topk_idx, topk_gate and logits are all NULL");
  if (logits && !aligned(logits, 16)) return fail(MOE_ERR_INVALID_ARG, "logits is not 16-byte aligned");
  if (flags & ~(uint32_t)MOE_FLAG_RENORM) return fail(MOE_ERR_UNSUPPORTED, "unknown flag bits 0x%x", flags);
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace pointer is NULL");
  if (!aligned(ws, 256)) return fail(MOE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  const size_t need = moe_prerouter_workspace_bytes(T, (int32_t)E, (int32_t)F);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  const size_t o_part = align256((size_t)T * F * 4), o_lg = o_part + align256((size_t)T * E * 4);
  float* act = at<float>(ws, 0);
  float* part = at<float>(ws, o_part);
  float* lg = logits ? logits : at<float>(ws, o_lg);
  float* raw = at<float>(ws, o_lg + align256((size_t)T * E * 4));
  const moe::HeadDev hd{(int)H, (int)E, (int)F, head->w1, head->b1, head->w2, head->b2, head->wl};
  return hip_status(moe::launch_prerouter(x, xtype, T, hd, cur, prev, k, (flags & MOE_FLAG_RENORM) ? 1 : 0, act, part,
                                          lg, topk_idx, topk_gate, raw, static_cast<hipStream_t>(stream)),
                    "prerouter head");
}

size_t moe_qlinear_lora_workspace_bytes(int32_t T, int32_t r) {
  if (T < 1 || T > 65536 || r < 0 || r > 64) return 0;
  return align256((size_t)T * (size_t)(r > 0 ? r : 1) * 4);
}

moe_status moe_qlinear_lora_forward(const void* x, int32_t xtype, int32_t T, const moe_qweight* w,
                                    const float* lora_a, const float* lora_b, int32_t r, float scale, float* y,
                                    void* ws, size_t ws_bytes, void* stream) {
  moe_status st;
  if ((st = check_x(x, xtype))) return st;
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weight struct is NULL");
  if (w->scheme != MOE_Q_SYM8 && w->scheme != MOE_Q_INT4)
    return fail(MOE_ERR_UNSUPPORTED, "unknown weight codec %d", w->scheme);
  if (T < 1 || T > 65536) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [1, 65536]", T);
  if (w->N < 1 || w->N > 65536) return fail(MOE_ERR_INVALID_ARG, "N=%d outside [1, 65536]", w->N);
  if (w->K < 32 || w->K > 4096 || w->K % 32)
    return fail(MOE_ERR_INVALID_ARG, "K=%d must be a multiple of 32 in [32, 4096]", w->K);
  if (r < 0 || r > 64) return fail(MOE_ERR_INVALID_ARG, "r=%d outside [0, 64]", r);
  if (!w->codes || !w->scales || !y) return fail(MOE_ERR_INVALID_ARG, "codes, scales or y is NULL");
  if (!aligned(w->codes, 16) || !aligned(w->scales, 2) || !aligned(y, 4))
    return fail(MOE_ERR_INVALID_ARG, "codes must be 16-byte aligned, scales 2-byte and y 4-byte aligned");
  if (r > 0 && (!lora_a || !lora_b)) return fail(MOE_ERR_INVALID_ARG, "lora_a or lora_b is NULL with r > 0");
  if (r > 0 && (!aligned(lora_a, 16) || !aligned(lora_b, 4)))
    return fail(MOE_ERR_INVALID_ARG, "lora_a must be 16-byte aligned and lora_b 4-byte aligned");
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace pointer is NULL");
  if (!aligned(ws, 256)) return fail(MOE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  const size_t need = moe_qlinear_lora_workspace_bytes(T, r);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return hip_status(moe::launch_qlinear_lora(x, xtype, T, w->N, w->K, w->scheme, static_cast<const uint8_t*>(w->codes),
                                             w->scales, lora_a, lora_b, r, scale, at<float>(ws, 0), y,
                                             static_cast<hipStream_t>(stream)),
                    "quantized linear with LoRA");
}

moe_status moe_prerouted_layer_forward(const void* x, int32_t xtype, int32_t T, const float* logits,
                                       const moe_experts* ex, int32_t k, uint32_t flags, float* y,
                                       int32_t* topk_idx_out, float* topk_gate_out, const moe_prerouter* head,
                                       const int32_t* prev_idx, float* logits_next, void* ws, size_t ws_bytes,
                                       void* stream) {
  moe_status st;
  moe::ExpertsDev d;
  Layout L;
  if ((st = check_layer_args(x, xtype, T, ex, k, flags, y, ws, ws_bytes, &d, &L))) return st;
  if (!logits) return fail(MOE_ERR_INVALID_ARG, "logits is NULL");
  if (!aligned(logits, 16)) return fail(MOE_ERR_INVALID_ARG, "logits is not 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!head) return layer_from_logits(x, xtype, T, d, k, flags, logits, 1, y, topk_idx_out, topk_gate_out, ws, L, s);
  if ((st = check_head(head, T, k))) return st;
  if (head->H != d.H || head->E != d.E)
    return fail(MOE_ERR_INVALID_ARG, "head (H=%d, E=%d) does not match the experts (H=%d, E=%d)", head->H, head->E,
                d.H, d.E);
  if (!topk_idx_out) return fail(MOE_ERR_INVALID_ARG, "topk_idx_out is NULL (the head reads this layer's routing)");
  if (!logits_next || !aligned(logits_next, 16))
    return fail(MOE_ERR_INVALID_ARG, "logits_next is NULL or not 16-byte aligned");
  if (prev_idx && !aligned(prev_idx, 4)) return fail(MOE_ERR_INVALID_ARG, "prev_idx is not 4-byte aligned");
  // the fused launches read these while they write the others
  if (prev_idx && prev_idx == topk_idx_out) return fail(MOE_ERR_INVALID_ARG, "prev_idx aliases topk_idx_out");
  if (logits_next == logits) return fail(MOE_ERR_INVALID_ARG, "logits_next aliases logits");
  const size_t base = align256(L.total);
  const size_t need = base + moe_prerouter_workspace_bytes(T, head->E, head->F);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  const moe::HeadDev hd{head->H, head->E, head->F, head->w1, head->b1, head->w2, head->b2, head->wl};
  float* act = at<float>(ws, base);
  float* part = at<float>(ws, base + align256((size_t)T * head->F * 4));
  float* raw = at<float>(ws, base + align256((size_t)T * head->F * 4) + 2 * align256((size_t)T * head->E * 4));
  const int renorm = (flags & MOE_FLAG_RENORM) ? 1 : 0;
  // (fp32 h is not a form of the fused launches: the expert and head launches run separately)
  if (T == 1 && !(flags & (MOE_FLAG_PATH_GEMM | MOE_FLAG_H_FP32)) && moe::prerouted_t1_fusable(d, xtype, hd))
    return hip_status(moe::launch_prerouted_t1(x, xtype, d, k, renorm, logits, at<int32_t>(ws, L.idx),
                                               at<float>(ws, L.gate), topk_idx_out, topk_gate_out,
                                               at<float>(ws, L.h), y, hd, prev_idx, act, part, logits_next, s),
                      "prerouted decode (one token)");
  if ((st = layer_from_logits(x, xtype, T, d, k, flags, logits, 1, y, topk_idx_out, topk_gate_out, ws, L, s)))
    return st;
  return hip_status(moe::launch_prerouter(x, xtype, T, hd, topk_idx_out, prev_idx, k, renorm, act, part, logits_next,
                                          nullptr, nullptr, raw, s),
                    "prerouter head");
}

moe_status moe_stream_read(const void* buf, int64_t bytes, void* stream) {
  if (!buf || !aligned(buf, 16)) return fail(MOE_ERR_INVALID_ARG, "buf is NULL or not 16-byte aligned");
  if (bytes <= 0 || bytes % 16 || bytes > ((int64_t)1 << 40))
    return fail(MOE_ERR_INVALID_ARG, "bytes=%lld: must be a positive multiple of 16, at most 2^40", (long long)bytes);
  return hip_status(moe::launch_stream_read(buf, bytes, static_cast<hipStream_t>(stream)), "stream read");
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_err.c_str(); }

}  // extern "C"
