// Prerouter head stages as device functions, shared by the head's own kernels
// and by the decode kernels that run the head beside the experts.
// "The Other Half of the Memory Wall: Serving 35B MoEs from SSD with Trained
// Routing Prediction" (xyznot.com), section 手法 (method), "Prerouterヘッドの
// アーキテクチャ": input [hidden ; k-hot current routing ; k-hot previous
// routing], head = fc2(erf-gelu(fc1(input))) + l(input).
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kHeadWaves = 4;

static __device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

// Stage 1, rows of two matrices in one launch. Rows r < R1 are fc1's
// (out1[t][r] = gelu(W1[r] . f_t + b1[r])); rows R1 + e are the residual
// path's (out2[t][e] = Wl[e] . f_t + b2[e], fc2's bias folded in here). Both
// matrices have rows of ldx = H + 2E values over f_t = [x_t ; khot(cur_t) ;
// khot(prev_t)]: the hidden part is a dot product, the k-hot part the sum of
// the row's entries at the 2k routed ids. blockIdx.y picks GROUPS groups of TU
// tokens; the row's hidden part stays in registers across them. Wave w owns
// the 256-column chunks w, w + 4, w + 8, ... of the hidden part.
// Run by a workgroup of kHeadWaves waves as block (bx, by) of that grid; cur may
// point to LDS.
template <int XT, int NCH, int TU, int GROUPS>
__device__ __forceinline__ void head_stage1_body(
    int bx, int by, const void* __restrict__ x, int T, int H, int E, int R1, const float* __restrict__ W1,
    const float* __restrict__ b1, const float* __restrict__ Wl, const float* __restrict__ b2,
    const int32_t* cur, const int32_t* __restrict__ prev, int k, float* __restrict__ out1,
    float* __restrict__ out2) {
  __shared__ float red[kHeadWaves][TU];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const bool fc1 = bx < R1;
  const int r = fc1 ? bx : bx - R1;
  const int t0 = by * TU * GROUPS;
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

// Stage 1 for one token inside the fused decode launch, which first picks the
// token's routing from the logits (the k-hot input). The row's reads that do
// not need it (its hidden part, the activations, the previous token's routed
// entries) go out first and stay in flight while wave 0 picks the routing;
// only the current token's k entries are read after it. The sums are
// head_stage1_body's, in the same order.
template <int XT, int NCH, int VPL>
__device__ __forceinline__ void head_stage1_t1_routed(int bx, const void* __restrict__ x, int H, int E, int R1,
                                                      const float* __restrict__ W1, const float* __restrict__ b1,
                                                      const float* __restrict__ Wl, const float* __restrict__ b2,
                                                      const float* __restrict__ logits, int k, int renorm,
                                                      const int32_t* __restrict__ prev, float* __restrict__ out1,
                                                      float* __restrict__ out2) {
  __shared__ float red[kHeadWaves];
  __shared__ int32_t cur_sh[kMaxK];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const bool fc1 = bx < R1;
  const int r = fc1 ? bx : bx - R1;
  const int64_t ldx = (int64_t)H + 2 * E;
  const float* wx = (fc1 ? W1 : Wl) + (int64_t)r * ldx;
  const int nx = (H + 255) >> 8;
  float4 wr[NCH], v[NCH];
  bool ok[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = w + kHeadWaves * i;
    const int j = c * 256 + lane * 4;
    ok[i] = c < nx && j < H;
    const int col = min(j, H - 4);  // in bounds; masked out of the sums when !ok
    wr[i] = c < nx ? *reinterpret_cast<const float4*>(wx + col) : make_float4(0.f, 0.f, 0.f, 0.f);
    v[i] = c < nx ? load_x4<XT>(x, col) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // lanes k .. 2k-1 of wave 0: the previous token's routed entries
  const float gp = (w == 0 && lane >= k && lane < 2 * k && prev) ? wx[H + E + prev[lane - k]] : 0.0f;
  if (w == 0) {
    int my_idx;
    float my_gate;
    wave_topk<VPL>(logits, E, k, renorm != 0, my_idx, my_gate, k, nullptr, 0, nullptr, false);  // ids only
    if (lane < k) cur_sh[lane] = my_idx;
  }
  __syncthreads();
  // lanes 0 .. k-1 of wave 0: the current token's routed entries
  float acc = (w == 0 && lane < k) ? wx[H + cur_sh[lane]] : gp;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (ok[i]) {
      acc = fmaf(wr[i].x, v[i].x, acc);
      acc = fmaf(wr[i].y, v[i].y, acc);
      acc = fmaf(wr[i].z, v[i].z, acc);
      acc = fmaf(wr[i].w, v[i].w, acc);
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) red[w] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float* bias = fc1 ? b1 : b2;
    float z = bias ? bias[r] : 0.0f;
#pragma unroll
    for (int q = 0; q < kHeadWaves; ++q) z += red[q];
    if (fc1) out1[r] = gelu_erf(z);
    else out2[r] = z;
  }
}

// Stage 2: logits[t][e] = part[t][e] + w2[e] . act_t, one wave per expert row
// (its F values in registers), nw rows per workgroup (its wave count), TU
// tokens per block row `by`.
template <int NCHF, int TU>
__device__ __forceinline__ void head_stage2_body(int bx, int by, int nw, const float* __restrict__ act,
                                                 const float* __restrict__ part, const float* __restrict__ w2, int T,
                                                 int E, int F, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = bx * nw + w;
  const int t0 = by * TU;
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

}  // namespace moe
