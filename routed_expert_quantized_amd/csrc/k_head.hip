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
// part in registers); fc2 needs all of fc1's outputs and is the second launch.
// The top-k follows as the router's one-wave kernel, or, for a few tokens of a
// narrow head, inside the second launch. A caller that hands the logits to the
// next layer's expert call skips it: that call takes the top-k inside its own
// first kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kHeadWaves = 4;

__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

// Stage 1, rows of two matrices in one launch. Rows r < R1 are fc1's
// (out1[t][r] = gelu(W1[r] . f_t + b1[r])); rows R1 + e are the residual
// path's (out2[t][e] = Wl[e] . f_t + b2[e], fc2's bias folded in here). Both
// matrices have rows of ldx = H + 2E values over f_t = [x_t ; khot(cur_t) ;
// khot(prev_t)]: the hidden part is a dot product, the k-hot part the sum of
// the row's entries at the 2k routed ids. blockIdx.y picks GROUPS groups of TU
// tokens; the row's hidden part stays in registers across them. Wave w owns
// the 256-column chunks w, w + 4, w + 8, ... of the hidden part.
template <int XT, int NCH, int TU, int GROUPS>
__global__ __launch_bounds__(64 * kHeadWaves) void k_head_stage1(
    const void* __restrict__ x, int T, int H, int E, int R1, const float* __restrict__ W1,
    const float* __restrict__ b1, const float* __restrict__ Wl, const float* __restrict__ b2,
    const int32_t* __restrict__ cur, const int32_t* __restrict__ prev, int k, float* __restrict__ out1,
    float* __restrict__ out2) {
  __shared__ float red[kHeadWaves][TU];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const bool fc1 = (int)blockIdx.x < R1;
  const int r = fc1 ? blockIdx.x : blockIdx.x - R1;
  const int t0 = blockIdx.y * TU * GROUPS;
  const int64_t ldx = (int64_t)H + 2 * E;
  const float* wx = (fc1 ? W1 : Wl) + (int64_t)r * ldx;
  const int nx = (H + 255) >> 8;
  float4 wr[NCH];
  int col[NCH];
  bool ok[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = w + kHeadWaves * i;
    const int j = c * 256 + lane * 4;
    ok[i] = c < nx && j < H;
    col[i] = min(j, H - 4);  // in bounds; masked out of the sums when !ok
    wr[i] = c < nx ? *reinterpret_cast<const float4*>(wx + col[i]) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // wave 0's lanes 0..2k-1 each add one routed column: lane j < k the current
  // token's j-th id, lane k + j the previous token's j-th id
  const bool gathers = w == 0 && lane < 2 * k;
  const int32_t* ids = lane < k ? cur : prev;
  const int slot = lane < k ? lane : lane - k;
  const int64_t base = (int64_t)H + (lane < k ? 0 : E);
  const int tend = min(t0 + TU * GROUPS, T);
  for (int tb = t0; tb < tend; tb += TU) {
    float4 v[TU][NCH];
    float g[TU];
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      const int t = min(tb + u, T - 1);
#pragma unroll
      for (int i = 0; i < NCH; ++i)
        v[u][i] = w + kHeadWaves * i < nx ? load_x4<XT>(x, (int64_t)t * H + col[i]) : make_float4(0.f, 0.f, 0.f, 0.f);
      g[u] = (gathers && ids) ? wx[base + ids[(int64_t)t * k + slot]] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      float acc = g[u];
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        if (ok[i]) {
          acc = fmaf(wr[i].x, v[u][i].x, acc);
          acc = fmaf(wr[i].y, v[u][i].y, acc);
          acc = fmaf(wr[i].z, v[u][i].z, acc);
          acc = fmaf(wr[i].w, v[u][i].w, acc);
        }
      }
      acc = wave_sum(acc);
      if (lane == 0) red[w][u] = acc;
    }
    __syncthreads();
    if (w == 0 && lane < TU && tb + lane < T) {
      const float* bias = fc1 ? b1 : b2;
      float z = bias ? bias[r] : 0.0f;
#pragma unroll
      for (int q = 0; q < kHeadWaves; ++q) z += red[q][lane];
      if (fc1) out1[(int64_t)(tb + lane) * R1 + r] = gelu_erf(z);
      else out2[(int64_t)(tb + lane) * E + r] = z;
    }
    __syncthreads();
  }
}

// Stage 2: logits[t][e] = part[t][e] + w2[e] . act_t, one wave per expert row
// (its F values in registers), kHeadWaves rows per workgroup, TU tokens per
// blockIdx.y. The router's one-wave top-k kernel follows.
template <int NCHF, int TU>
__global__ __launch_bounds__(64 * kHeadWaves) void k_head_stage2(
    const float* __restrict__ act, const float* __restrict__ part, const float* __restrict__ w2, int T, int E,
    int F, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blockIdx.x * kHeadWaves + w;
  const int t0 = blockIdx.y * TU;
  if (e >= E) return;
  const float* row = w2 + (int64_t)e * F;
  float4 wr[NCHF];
  int col[NCHF];
  bool ok[NCHF];
#pragma unroll
  for (int i = 0; i < NCHF; ++i) {
    const int j = i * 256 + lane * 4;
    ok[i] = j < F;
    col[i] = min(j, F - 4);
    wr[i] = *reinterpret_cast<const float4*>(row + col[i]);
  }
  float4 v[TU][NCHF];
#pragma unroll
  for (int u = 0; u < TU; ++u) {
    const int t = min(t0 + u, T - 1);
#pragma unroll
    for (int i = 0; i < NCHF; ++i) v[u][i] = *reinterpret_cast<const float4*>(act + (int64_t)t * F + col[i]);
  }
#pragma unroll
  for (int u = 0; u < TU; ++u) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < NCHF; ++i) {
      if (ok[i]) {
        acc = fmaf(wr[i].x, v[u][i].x, acc);
        acc = fmaf(wr[i].y, v[u][i].y, acc);
        acc = fmaf(wr[i].z, v[u][i].z, acc);
        acc = fmaf(wr[i].w, v[u][i].w, acc);
      }
    }
    acc = wave_sum(acc);
    const int t = t0 + u;
    if (lane == 0 && t < T) logits[(int64_t)t * E + e] = part[(int64_t)t * E + e] + acc;
  }
}

// Stage 2 with the top-k, for a few tokens of a narrow head (F <= 256, E <=
// kFuseWaves * kFuseRows): one 1024-thread workgroup per token. Wave w takes
// rows w, w + 16, ...; every lane issues all its row loads before the first
// sum, so the whole of fc2 is in flight at once. The E logits land in LDS and
// wave 0 runs the router's top-k on them; they also go out to memory.
constexpr int kFuseTopkMaxT = 4;
constexpr int kFuseWaves = 16;
constexpr int kFuseRows = 16;

template <int RPW, int VPL>
__global__ __launch_bounds__(64 * kFuseWaves) void k_head_stage2_topk(
    const float* __restrict__ act, const float* __restrict__ part, const float* __restrict__ w2, int E, int F,
    float* __restrict__ logits, int k, int renorm, int32_t* __restrict__ idx, float* __restrict__ gate) {
  __shared__ float lg[64 * VPL];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x;
  const bool ok = lane * 4 < F;
  const int col = min(lane * 4, F - 4);
  const float4 v = *reinterpret_cast<const float4*>(act + (int64_t)t * F + col);
  float4 r[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int e = min(w + kFuseWaves * i, E - 1);
    r[i] = *reinterpret_cast<const float4*>(w2 + (int64_t)e * F + col);
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int e = w + kFuseWaves * i;
    float acc = 0.0f;
    if (ok) {
      acc = fmaf(r[i].x, v.x, acc);
      acc = fmaf(r[i].y, v.y, acc);
      acc = fmaf(r[i].z, v.z, acc);
      acc = fmaf(r[i].w, v.w, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0 && e < E) {
      const float z = part[(int64_t)t * E + e] + acc;
      lg[e] = z;
      logits[(int64_t)t * E + e] = z;
    }
  }
  __syncthreads();
  if (w == 0) {
    int my_idx;
    float my_gate;
    wave_topk<VPL>(lg, E, k, renorm != 0, my_idx, my_gate);
    if (lane < k) {
      idx[(int64_t)t * k + lane] = my_idx;
      gate[(int64_t)t * k + lane] = my_gate;
    }
  }
}

}  // namespace

hipError_t launch_prerouter(const void* x, int xtype, int T, const HeadDev& hd, const int32_t* cur,
                            const int32_t* prev, int k, int renorm, float* act, float* part, float* logits,
                            int32_t* idx, float* gate, hipStream_t s) {
  const int H = hd.H, E = hd.E, F = hd.F;
  // stage 1: a = gelu(fc1(f)) for F rows, part = l(f) + b2 for E rows
  {
    const int nch = ((H + 255) / 256 + kHeadWaves - 1) / kHeadWaves;
    // groups of 4 tokens per workgroup: enough workgroups to fill the GPU,
    // few enough re-reads of each weight row
    const int groups = T <= 16 ? 1 : T <= 64 ? 4 : 8;
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
      else if (groups == 1) go(NC, I4{}, I1{});
      else if (groups == 4) go(NC, I4{}, I4{});
      else go(NC, I4{}, std::integral_constant<int, 8>{});
    };
    if (nch <= 1) with_tu(std::integral_constant<int, 1>{});
    else if (nch <= 2) with_tu(std::integral_constant<int, 2>{});
    else with_tu(std::integral_constant<int, 4>{});
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // stage 2: logits = part + fc2(a), then the top-k (in the same kernel for a few tokens)
  const int nchf = (F + 255) / 256;
  auto with_nchf = [&](auto fn) {
    if (nchf <= 1) fn(std::integral_constant<int, 1>{});
    else if (nchf <= 2) fn(std::integral_constant<int, 2>{});
    else if (nchf <= 4) fn(std::integral_constant<int, 4>{});
    else if (nchf <= 8) fn(std::integral_constant<int, 8>{});
    else fn(std::integral_constant<int, 16>{});
  };
  if (idx && T <= kFuseTopkMaxT && F <= 256 && E <= kFuseWaves * kFuseRows) {
    const int rpw = (E + kFuseWaves - 1) / kFuseWaves;
    const int vpl = (E + 63) / 64;
    auto go = [&](auto RC, auto VC) {
      constexpr int R = decltype(RC)::value, V = decltype(VC)::value;
      MOE_LAUNCH(MOE_KERNEL_HEAD, (k_head_stage2_topk<R, V>), dim3(T), dim3(64 * kFuseWaves), 0, s, act, part, hd.w2,
                 E, F, logits, k, renorm, idx, gate);
    };
    if (rpw <= 1) go(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
    else if (rpw <= 4) go(std::integral_constant<int, 4>{}, std::integral_constant<int, 1>{});
    else if (vpl <= 2) go(std::integral_constant<int, 8>{}, std::integral_constant<int, 2>{});
    else go(std::integral_constant<int, kFuseRows>{}, std::integral_constant<int, 4>{});
    return hipGetLastError();
  }
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
