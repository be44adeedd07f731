// k_route.hip — router kernels: logits GEMV/GEMM, one-wave top-k, token-by-expert grouping.
//
// [LR] "QwenのMoEルーターを観測してホットエキスパートを先読みしても速くならなかった" (lilting.ch),
//      section "ルーターをフックする": the router is a gate linear, a softmax and a top-k.
#include <type_traits>

#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------- logits, few tokens
// One wave per expert row: logits[t][e] = R[e] . x[t] in fp32, for every token.
// The row is loaded once into registers (NCH float4 chunks per lane, all loads
// issued together) and reused for each token; tokens go TU at a time with
// their activation loads issued before any arithmetic.
template <int XT, int NCH, int TU>
__global__ __launch_bounds__(64) void k_logits_rows(const void* __restrict__ x, int T, int H,
                                                    const float* __restrict__ R, int E,
                                                    float* __restrict__ logits) {
  const int lane = threadIdx.x;
  const int e = blockIdx.x;
  const float* row = R + (int64_t)e * H;
  float4 r[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = min(lane * 4 + 256 * c, H - 4);
    r[c] = *reinterpret_cast<const float4*>(row + i);
  }
  for (int t0 = 0; t0 < T; t0 += TU) {
    float4 v[TU][NCH];
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      const int t = min(t0 + u, T - 1);
#pragma unroll
      for (int c = 0; c < NCH; ++c) v[u][c] = load_x4<XT>(x, (int64_t)t * H + min(lane * 4 + 256 * c, H - 4));
    }
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (lane * 4 + 256 * c < H) {
          acc = fmaf(r[c].x, v[u][c].x, acc);
          acc = fmaf(r[c].y, v[u][c].y, acc);
          acc = fmaf(r[c].z, v[u][c].z, acc);
          acc = fmaf(r[c].w, v[u][c].w, acc);
        }
      }
      acc = wave_sum(acc);
      if (lane == 0 && t0 + u < T) logits[(int64_t)(t0 + u) * E + e] = acc;
    }
  }
}

// ---------------------------------------------------------------- logits, many tokens
// Tiled fp32 GEMM logits[T][E] = X[T][H] R[E][H]^T: 64x64 output tile per
// workgroup, K steps of 16 staged in LDS, 4x4 outputs per thread.
template <int XT>
__global__ __launch_bounds__(256) void k_logits_tiled(const void* __restrict__ x, int T, int H,
                                                      const float* __restrict__ R, int E,
                                                      float* __restrict__ logits) {
  __shared__ float xs[16][64 + 4];
  __shared__ float rs[16][64 + 4];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tx = tid & 15, ty = tid >> 4;  // outputs (t0 + ty*4 + i, e0 + tx*4 + j)
  float acc[4][4] = {};
  // loader: 256 threads load 64 rows x 16 columns = 4 elements each
  const int lr = tid >> 2, lc = (tid & 3) * 4;
  for (int h0 = 0; h0 < H; h0 += 16) {
    {
      const int t = t0 + lr;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < T) v = load_x4<XT>(x, (int64_t)t * H + h0 + lc);
      xs[lc + 0][lr] = v.x; xs[lc + 1][lr] = v.y; xs[lc + 2][lr] = v.z; xs[lc + 3][lr] = v.w;
      const int e = e0 + lr;
      float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < E) r = *reinterpret_cast<const float4*>(R + (int64_t)e * H + h0 + lc);
      rs[lc + 0][lr] = r.x; rs[lc + 1][lr] = r.y; rs[lc + 2][lr] = r.z; rs[lc + 3][lr] = r.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = xs[kk][ty * 4 + i]; b[i] = rs[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) logits[(int64_t)t * E + e] = acc[i][j];
    }
  }
}

// ---------------------------------------------------------------- top-k, one wave per token
template <int VPL>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int renorm, int32_t* __restrict__ idx, float* __restrict__ gate,
                                              int32_t* __restrict__ idx2, float* __restrict__ gate2) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  int my_idx;
  float my_gate;
  wave_topk<VPL>(logits + (int64_t)t * E, E, k, renorm != 0, my_idx, my_gate);
  if (lane < k) {
    idx[(int64_t)t * k + lane] = my_idx;
    gate[(int64_t)t * k + lane] = my_gate;
    if (idx2) idx2[(int64_t)t * k + lane] = my_idx;
    if (gate2) gate2[(int64_t)t * k + lane] = my_gate;
  }
}

// ---------------------------------------------------------------- grouping
// Tokens are cut into chunks of 64. For chunk c and expert e, mask[c][e] has
// bit (t mod 64) set when token t routes to e. A token's k experts are
// distinct, so the stable position of assignment (t, e) in expert e's list is
// the number of earlier set bits: in earlier chunks (base[c][e]) and below
// bit t in its own word.
__global__ __launch_bounds__(256) void k_group_mask(const int32_t* __restrict__ idx, int T, int k, int E,
                                                    uint64_t* __restrict__ mask) {
  __shared__ unsigned long long m[kMaxE];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) m[e] = 0ull;
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * k; i += 256) {
    const int t = c * 64 + i / k;
    if (t < T) atomicOr(&m[idx[(int64_t)t * k + (i % k)]], 1ull << (t & 63));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) mask[(int64_t)c * E + e] = m[e];
}

// Exclusive scan over a 1024-thread block; returns the prefix and the total.
__device__ __forceinline__ int block_exclusive_scan_1024(int v, int* smem, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) smem[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? smem[lane] : 0;
    int wi = w;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(wi, off, 64);
      if (lane >= off) wi += o;
    }
    if (lane < 16) smem[16 + lane] = wi - w;  // exclusive prefix of wave totals
    if (lane == 15) smem[32] = wi;
  }
  __syncthreads();
  const int excl = incl - v + smem[16 + wave];
  total = smem[32];
  __syncthreads();
  return excl;
}

__global__ __launch_bounds__(1024) void k_group_scan(const uint64_t* __restrict__ mask, int C, int E,
                                                     int32_t* __restrict__ base, int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ uniq,
                                                     int32_t* __restrict__ n_uniq) {
  __shared__ int smem[64];
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E) {
    for (int c = 0; c < C; ++c) {
      base[(int64_t)c * E + e] = cnt;
      cnt += __popcll(mask[(int64_t)c * E + e]);
    }
    counts[e] = cnt;
  }
  int total;
  const int off = block_exclusive_scan_1024(cnt, smem, total);
  if (e < E) {
    offsets[e] = off;
    for (int c = 0; c < C; ++c) base[(int64_t)c * E + e] += off;
  }
  if (e == 0) offsets[E] = total;
  int nu;
  const int pos = block_exclusive_scan_1024(cnt > 0 ? 1 : 0, smem, nu);
  if (e < E && cnt > 0) uniq[pos] = e;
  if (e == 0) *n_uniq = nu;
}

__global__ __launch_bounds__(256) void k_group_scatter(const int32_t* __restrict__ idx, int T, int k, int E,
                                                       const uint64_t* __restrict__ mask,
                                                       const int32_t* __restrict__ base,
                                                       int32_t* __restrict__ perm) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (f >= (int64_t)T * k) return;
  const int t = (int)(f / k);
  const int e = idx[f];
  const int c = t >> 6, bit = t & 63;
  const uint64_t below = bit ? (mask[(int64_t)c * E + e] & ((1ull << bit) - 1ull)) : 0ull;
  perm[base[(int64_t)c * E + e] + __popcll(below)] = (int32_t)f;
}

// ---------------------------------------------------------------- launchers
hipError_t launch_logits(const void* x, int xtype, int T, int H, const float* R, int E, float* logits,
                         hipStream_t s) {
  if (T >= kTiledLogitsMinT) {
    dim3 grid((T + 63) / 64, (E + 63) / 64);
    switch (xtype) {
      case MOE_F32: MOE_LAUNCH(MOE_KERNEL_ROUTE_LOGITS, k_logits_tiled<MOE_F32>, grid, dim3(256), 0, s, x, T, H, R, E, logits); break;
      case MOE_F16: MOE_LAUNCH(MOE_KERNEL_ROUTE_LOGITS, k_logits_tiled<MOE_F16>, grid, dim3(256), 0, s, x, T, H, R, E, logits); break;
      default:      MOE_LAUNCH(MOE_KERNEL_ROUTE_LOGITS, k_logits_tiled<MOE_BF16>, grid, dim3(256), 0, s, x, T, H, R, E, logits); break;
    }
  } else {
    const int nch = (H + 255) / 256;
    auto go = [&](auto NC) {
      constexpr int N = decltype(NC)::value;
      constexpr int TU = N >= 16 ? 2 : N >= 8 ? 4 : 8;
      switch (xtype) {
        case MOE_F32: MOE_LAUNCH(MOE_KERNEL_ROUTE_LOGITS, (k_logits_rows<MOE_F32, N, TU>), dim3(E), dim3(64), 0, s, x, T, H, R, E, logits); break;
        case MOE_F16: MOE_LAUNCH(MOE_KERNEL_ROUTE_LOGITS, (k_logits_rows<MOE_F16, N, TU>), dim3(E), dim3(64), 0, s, x, T, H, R, E, logits); break;
        default:      MOE_LAUNCH(MOE_KERNEL_ROUTE_LOGITS, (k_logits_rows<MOE_BF16, N, TU>), dim3(E), dim3(64), 0, s, x, T, H, R, E, logits); break;
      }
    };
    if (nch <= 1) go(std::integral_constant<int, 1>{});
    else if (nch <= 2) go(std::integral_constant<int, 2>{});
    else if (nch <= 4) go(std::integral_constant<int, 4>{});
    else if (nch <= 8) go(std::integral_constant<int, 8>{});
    else go(std::integral_constant<int, 16>{});
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int renorm, int32_t* idx, float* gate,
                       int32_t* idx2, float* gate2, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  const int vpl = (E + 63) / 64;
  if (vpl <= 1)      MOE_LAUNCH(MOE_KERNEL_TOPK, k_topk<1>, grid, dim3(256), 0, s, logits, T, E, k, renorm, idx, gate, idx2, gate2);
  else if (vpl <= 2) MOE_LAUNCH(MOE_KERNEL_TOPK, k_topk<2>, grid, dim3(256), 0, s, logits, T, E, k, renorm, idx, gate, idx2, gate2);
  else if (vpl <= 4) MOE_LAUNCH(MOE_KERNEL_TOPK, k_topk<4>, grid, dim3(256), 0, s, logits, T, E, k, renorm, idx, gate, idx2, gate2);
  else if (vpl <= 8) MOE_LAUNCH(MOE_KERNEL_TOPK, k_topk<8>, grid, dim3(256), 0, s, logits, T, E, k, renorm, idx, gate, idx2, gate2);
  else               MOE_LAUNCH(MOE_KERNEL_TOPK, k_topk<16>, grid, dim3(256), 0, s, logits, T, E, k, renorm, idx, gate, idx2, gate2);
  return hipGetLastError();
}

hipError_t launch_group(const int32_t* idx, int T, int k, int E, const GroupBufs& g, hipStream_t s) {
  const int C = (T + 63) / 64;
  MOE_LAUNCH(MOE_KERNEL_GROUP, k_group_mask, dim3(C), dim3(256), 0, s, idx, T, k, E, g.mask);
  MOE_LAUNCH(MOE_KERNEL_GROUP, k_group_scan, dim3(1), dim3(1024), 0, s, g.mask, C, E, g.base, g.counts, g.offsets, g.uniq,
                     g.n_uniq);
  const int64_t n = (int64_t)T * k;
  MOE_LAUNCH(MOE_KERNEL_GROUP, k_group_scatter, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, idx, T, k, E, g.mask,
                     g.base, g.perm);
  return hipGetLastError();
}

}  // namespace moe
