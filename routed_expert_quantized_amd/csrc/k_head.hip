// Prerouter head: a small two-layer network with a linear residual path that,
// run at one layer, gives the routing of the next layer for the next token.
// "The Other Half of the Memory Wall: Serving 35B MoEs from SSD with Trained
// Routing Prediction" (xyznot.com), section 手法 (method), "Prerouterヘッドの
// アーキテクチャ": the input is the hidden state joined with the k-hot routing
// vectors of the current and the previous token (H + 2E values), and the head
// is fc2(erf-gelu(fc1(input))) plus a linear path warm-started from the next
// layer's router; section 主なアイデア (prediction as routing): its top-k is the
// routing.
//
// The k-hot part of the input is never built: a weight row's product with it is
// the sum of the 2k entries at the routed ids, gathered from the row itself.
// fc1 and the residual path both read the whole input, so they share the first
// launch (one workgroup per output row and group of tokens, the row's hidden
// part in registers); from 16 tokens the hidden-part products run instead on
// the fp32 matrix cores (the router's logits kernel) and a small epilogue adds
// the routed columns, the biases and the GELU. fc2 needs all of fc1's outputs
// and is the next launch. The top-k follows as the router's one-wave kernel; a
// caller that hands the logits to the next layer's expert call skips it, since
// that call takes the top-k inside its own first kernel.
#include "common.hpp"
#include "head_rows.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

template <int XT, int NCH, int TU, int GROUPS>
__global__ __launch_bounds__(64 * kHeadWaves) void k_head_stage1(
    const void* __restrict__ x, int T, int H, int E, int R1, const float* __restrict__ W1,
    const float* __restrict__ b1, const float* __restrict__ Wl, const float* __restrict__ b2,
    const int32_t* __restrict__ cur, const int32_t* __restrict__ prev, int k, float* __restrict__ out1,
    float* __restrict__ out2) {
  head_stage1_body<XT, NCH, TU, GROUPS>(blockIdx.x, blockIdx.y, x, T, H, E, R1, W1, b1, Wl, b2, cur, prev, k, out1,
                                        out2);
}

template <int NCHF, int TU>
__global__ __launch_bounds__(64 * kHeadWaves) void k_head_stage2(
    const float* __restrict__ act, const float* __restrict__ part, const float* __restrict__ w2, int T, int E,
    int F, float* __restrict__ logits) {
  head_stage2_body<NCHF, TU>(blockIdx.x, blockIdx.y, kHeadWaves, act, part, w2, T, E, F, logits);
}

// Stage 1 of a batch from the matrix-core products: the partial planes of
// W1 x (nsplit1 planes [T][ld1]) and Wl x (nsplit2 planes [T][ld2], from column
// off2) are added in plane order, then the k-hot columns and the bias, and
// fc1's rows take the GELU. One thread per (token, row). When the two matrices
// were one launch, both point at the same planes of F + E columns.
__global__ __launch_bounds__(256) void k_head_epilogue(const float* __restrict__ raw1, int nsplit1, int ld1,
                                                       const float* __restrict__ raw2, int nsplit2, int ld2, int off2,
                                                       int T, int H, int E, int F, const float* __restrict__ W1,
                                                       const float* __restrict__ b1, const float* __restrict__ Wl,
                                                       const float* __restrict__ b2, const int32_t* __restrict__ cur,
                                                       const int32_t* __restrict__ prev, int k,
                                                       float* __restrict__ act, float* __restrict__ part) {
  const int nbx = (F + E + 255) / 256;
  const int t = blockIdx.x / nbx;
  const int i = (blockIdx.x % nbx) * 256 + threadIdx.x;
  if (i >= F + E) return;
  const bool fc1 = i < F;
  const int r = fc1 ? i : i - F;
  const int R = fc1 ? ld1 : ld2;            // row length of the planes
  const float* raw = fc1 ? raw1 : raw2 + off2;
  const int ns = fc1 ? nsplit1 : nsplit2;
  const int64_t plane = (int64_t)T * R;
  // every load is issued before the first add: the planes, the routed ids,
  // then the routed columns
  float pz[kMaxLogitSplits];
#pragma unroll
  for (int q = 0; q < kMaxLogitSplits; ++q) pz[q] = q < ns ? raw[q * plane + (int64_t)t * R + r] : 0.0f;
  const float* row = (fc1 ? W1 : Wl) + (int64_t)r * (H + 2 * E);
  int id[2 * kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    id[j] = (cur && j < k) ? cur[(int64_t)t * k + j] : -1;
    id[kMaxK + j] = (prev && j < k) ? E + prev[(int64_t)t * k + j] : -1;
  }
  float gv[2 * kMaxK];
#pragma unroll
  for (int j = 0; j < 2 * kMaxK; ++j) gv[j] = id[j] >= 0 ? row[H + id[j]] : 0.0f;
  float z = pz[0];
#pragma unroll
  for (int q = 1; q < kMaxLogitSplits; ++q) z += pz[q];
  float g = 0.0f;
#pragma unroll
  for (int j = 0; j < 2 * kMaxK; ++j) g += gv[j];
  z += g;
  const float* bias = fc1 ? b1 : b2;
  if (bias) z += bias[r];
  if (fc1) act[(int64_t)t * F + r] = gelu_erf(z);
  else part[(int64_t)t * E + r] = z;
}

}  // namespace

hipError_t launch_prerouter(const void* x, int xtype, int T, const HeadDev& hd, const int32_t* cur,
                            const int32_t* prev, int k, int renorm, float* act, float* part, float* logits,
                            int32_t* idx, float* gate, float* raw, hipStream_t s) {
  const int H = hd.H, E = hd.E, F = hd.F;
  hipError_t e;
  if (T >= kMfmaLogitsMinT) {
    // a batch: the hidden-part products on the fp32 matrix cores (the router's
    // logits kernel with the head's row stride), then the epilogue
    const int64_t ldx = (int64_t)H + 2 * E;
    float* raw1 = raw;
    float* raw2 = raw + logits_max_splits(T, F) * (int64_t)T * F;
    int ns1 = 1, ns2 = 1, ld1 = F, ld2 = E, off2 = 0;
    if (hd.wl == hd.w1 + (int64_t)F * ldx) {
      // the residual path's rows follow fc1's in memory: one launch over F + E rows
      e = launch_logits(x, xtype, T, H, hd.w1, F + E, raw1, &ns1, false, s, ldx);
      if (e != hipSuccess) return e;
      raw2 = raw1;
      ns2 = ns1;
      ld1 = ld2 = F + E;
      off2 = F;
    } else {
      e = launch_logits(x, xtype, T, H, hd.w1, F, raw1, &ns1, false, s, ldx);
      if (e != hipSuccess) return e;
      e = launch_logits(x, xtype, T, H, hd.wl, E, raw2, &ns2, false, s, ldx);
      if (e != hipSuccess) return e;
    }
    MOE_LAUNCH(MOE_KERNEL_HEAD, k_head_epilogue, dim3((unsigned)(((F + E + 255) / 256) * T)), dim3(256), 0, s, raw1, ns1,
               ld1, raw2, ns2, ld2, off2, T,
               H, E, F, hd.w1, hd.b1, hd.wl, hd.b2, cur, prev, k, act, part);
  } else {
    // stage 1 of a few tokens: a = gelu(fc1(f)) for F rows, part = l(f) + b2 for
    // E rows, one workgroup per row and group of 4 tokens
    const int nch = ((H + 255) / 256 + kHeadWaves - 1) / kHeadWaves;
    auto go = [&](auto NC, auto TUc, auto GC) {
      constexpr int N = decltype(NC)::value, U = decltype(TUc)::value, G = decltype(GC)::value;
      const dim3 grid(F + E, (T + U * G - 1) / (U * G)), block(64 * kHeadWaves);
      switch (xtype) {
        case MOE_F32: MOE_LAUNCH(MOE_KERNEL_HEAD, (k_head_stage1<MOE_F32, N, U, G>), grid, block, 0, s, x, T, H, E, F, hd.w1, hd.b1, hd.wl, hd.b2, cur, prev, k, act, part); break;
        case MOE_F16: MOE_LAUNCH(MOE_KERNEL_HEAD, (k_head_stage1<MOE_F16, N, U, G>), grid, block, 0, s, x, T, H, E, F, hd.w1, hd.b1, hd.wl, hd.b2, cur, prev, k, act, part); break;
        default:      MOE_LAUNCH(MOE_KERNEL_HEAD, (k_head_stage1<MOE_BF16, N, U, G>), grid, block, 0, s, x, T, H, E, F, hd.w1, hd.b1, hd.wl, hd.b2, cur, prev, k, act, part); break;
      }
    };
    auto with_tu = [&](auto NC) {
      using I1 = std::integral_constant<int, 1>;
      using I4 = std::integral_constant<int, 4>;
      if (T == 1) go(NC, I1{}, I1{});
      else go(NC, I4{}, I1{});
    };
    if (nch <= 1) with_tu(std::integral_constant<int, 1>{});
    else if (nch <= 2) with_tu(std::integral_constant<int, 2>{});
    else with_tu(std::integral_constant<int, 4>{});
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // stage 2: logits = part + fc2(a), then the router's top-k
  const int nchf = (F + 255) / 256;
  auto with_nchf = [&](auto fn) {
    if (nchf <= 1) fn(std::integral_constant<int, 1>{});
    else if (nchf <= 2) fn(std::integral_constant<int, 2>{});
    else if (nchf <= 4) fn(std::integral_constant<int, 4>{});
    else if (nchf <= 8) fn(std::integral_constant<int, 8>{});
    else fn(std::integral_constant<int, 16>{});
  };
  with_nchf([&](auto NC) {
    constexpr int N = decltype(NC)::value;
    constexpr int U = N >= 8 ? 1 : N >= 4 ? 2 : 4;  // tokens per workgroup, within the register budget
    const dim3 grid((E + kHeadWaves - 1) / kHeadWaves, (T + U - 1) / U), block(64 * kHeadWaves);
    MOE_LAUNCH(MOE_KERNEL_HEAD, (k_head_stage2<N, U>), grid, block, 0, s, act, part, hd.w2, T, E, F, logits);
  });
  e = hipGetLastError();
  if (e != hipSuccess || !idx) return e;
  return launch_topk(logits, 1, T, E, k, renorm, idx, gate, nullptr, nullptr, s);
}

}  // namespace moe
