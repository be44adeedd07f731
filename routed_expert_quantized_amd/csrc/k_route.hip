// k_route.hip — router kernels: logits GEMV/GEMM, one-wave top-k, token-by-expert grouping.
//
// [LR] "QwenのMoEルーターを観測してホットエキスパートを先読みしても速くならなかった" (lilting.ch),
//      section "ルーターをフックする": the router is a gate linear, a softmax and a top-k.
#include <type_traits>
#include <utility>

#include "kernels.hpp"
#include "stamps.hpp"

namespace moe {

// timestamp build only: start and end of each row kernel workgroup
MOE_STAMP_TABLE(g_stamps_route, 2);

// ---------------------------------------------------------------- logits, few tokens
// WPE waves per expert row: logits[t][e] = R[e] . x[t] in fp32, for every token.
// Wave w owns the columns of chunks [w NCH, (w+1) NCH) (a chunk is 256
// columns, 4 per lane). Its part of the row is loaded once into registers (all
// loads issued together) and reused for each token; tokens go TU at a time with
// their activation loads issued before any arithmetic. The waves' partial sums
// meet in LDS and are added in wave order.
template <int XT, int NCH, int TU, int WPE>
__global__ __launch_bounds__(64 * WPE) void k_logits_rows(const void* __restrict__ x, int T, int H,
                                                          const float* __restrict__ R, int E,
                                                          float* __restrict__ logits) {
  __shared__ float red[WPE][TU];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blockIdx.x;
  MOE_STAMP(g_stamps_route, 0, blockIdx.x);
  const int c0 = w * NCH;
  const float* row = R + (int64_t)e * H;
  float4 r[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = min(lane * 4 + 256 * (c0 + c), H - 4);
    r[c] = *reinterpret_cast<const float4*>(row + i);
  }
  for (int t0 = 0; t0 < T; t0 += TU) {
    float4 v[TU][NCH];
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      const int t = min(t0 + u, T - 1);
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        v[u][c] = load_x4<XT>(x, (int64_t)t * H + min(lane * 4 + 256 * (c0 + c), H - 4));
    }
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (lane * 4 + 256 * (c0 + c) < H) {
          acc = fmaf(r[c].x, v[u][c].x, acc);
          acc = fmaf(r[c].y, v[u][c].y, acc);
          acc = fmaf(r[c].z, v[u][c].z, acc);
          acc = fmaf(r[c].w, v[u][c].w, acc);
        }
      }
      acc = wave_sum(acc);
      if constexpr (WPE == 1) {
        if (lane == 0 && t0 + u < T) logits[(int64_t)(t0 + u) * E + e] = acc;
      } else if (lane == 0) {
        red[w][u] = acc;
      }
    }
    if constexpr (WPE > 1) {
      __syncthreads();
      if (w == 0 && lane < TU && t0 + lane < T) {
        float acc = red[0][lane];
#pragma unroll
        for (int q = 1; q < WPE; ++q) acc += red[q][lane];
        logits[(int64_t)(t0 + lane) * E + e] = acc;
      }
      __syncthreads();
    }
  }
  MOE_STAMP(g_stamps_route, 1, blockIdx.x);
}

// ---------------------------------------------------------------- top-k, one wave per token
// With nsplit > 1 the logits arrive as split-K partial planes [nsplit][T][E];
// the wave first adds them, in plane order, into its own LDS row.
template <int VPL>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int nsplit, int T, int E, int k,
                                              int renorm, int32_t* __restrict__ idx, float* __restrict__ gate,
                                              int32_t* __restrict__ idx2, float* __restrict__ gate2) {
  __shared__ float lsum[4][64 * VPL];
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const float* row = logits + (int64_t)t * E;
  if (nsplit > 1) {
    // the loads of every plane for all of the lane's logits go out together,
    // then are added in plane order
    const int64_t plane = (int64_t)T * E;
    float p[kMaxLogitSplits][VPL];
#pragma unroll
    for (int q = 0; q < kMaxLogitSplits; ++q)
#pragma unroll
      for (int j = 0; j < VPL; ++j)
        p[q][j] = (q < nsplit && lane + 64 * j < E) ? row[q * plane + lane + 64 * j] : 0.0f;
    float v[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      v[j] = p[0][j];
#pragma unroll
      for (int q = 1; q < kMaxLogitSplits; ++q)
        if (q < nsplit) v[j] += p[q][j];
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (lane + 64 * j < E) lsum[wv][lane + 64 * j] = v[j];
    row = lsum[wv];  // written and read by this wave only, in order
  }
  int my_idx;
  float my_gate;
  wave_topk<VPL>(row, E, k, renorm != 0, my_idx, my_gate);
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

// Per expert e: counts[e], offsets[e] (exclusive scan of the counts), and
// base[c][e] = offsets[e] + the assignments of e in chunks before c. The
// 1024 threads split each expert's C chunks into P = 1024 / E parts (one
// thread per expert and part): each part counts its chunks, the parts' counts
// give every part its starting position, and each part then writes its
// chunks' bases, reading the masks again (batched) instead of updating the
// bases in place.
__global__ __launch_bounds__(1024) void k_group_scan(const uint64_t* __restrict__ mask, int C, int E,
                                                     int32_t* __restrict__ base, int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ uniq,
                                                     int32_t* __restrict__ n_uniq) {
  __shared__ int smem[64];
  __shared__ int part_cnt[1024];
  __shared__ int start[1024];
  const int P = 1024 / E;  // E <= 1024
  const int e = (int)threadIdx.x % E, p = (int)threadIdx.x / E;
  const bool active = p < P;
  const int c_lo = active ? (int)((int64_t)p * C / P) : 0, c_hi = active ? (int)((int64_t)(p + 1) * C / P) : 0;
  // masks of 8 chunks requested together
  auto for_chunks = [&](auto&& f) {
    for (int c0 = c_lo; c0 < c_hi; c0 += 8) {
      uint64_t mk[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) mk[j] = c0 + j < c_hi ? mask[(int64_t)(c0 + j) * E + e] : 0ull;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (c0 + j < c_hi) f(c0 + j, __popcll(mk[j]));
    }
  };
  int mine = 0;
  for_chunks([&](int, int n) { mine += n; });
  part_cnt[threadIdx.x] = mine;
  __syncthreads();
  int cnt = 0;  // the expert's count, on its part-0 thread
  if (p == 0)
    for (int q = 0; q < P; ++q) cnt += part_cnt[q * E + e];
  int total;
  const int off = block_exclusive_scan_1024(p == 0 ? cnt : 0, smem, total);
  if (p == 0) {
    counts[e] = cnt;
    offsets[e] = off;
    int run = off;  // each part's first position
    for (int q = 0; q < P; ++q) {
      start[q * E + e] = run;
      run += part_cnt[q * E + e];
    }
  }
  if (threadIdx.x == 0) offsets[E] = total;
  __syncthreads();
  if (active) {
    int run = start[threadIdx.x];
    for_chunks([&](int c, int n) {
      base[(int64_t)c * E + e] = run;
      run += n;
    });
  }
  int nu;
  const int pos = block_exclusive_scan_1024(p == 0 && cnt > 0 ? 1 : 0, smem, nu);
  if (p == 0 && cnt > 0) uniq[pos] = e;
  if (threadIdx.x == 0) *n_uniq = nu;
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

// The same grouping in one workgroup when the chunk masks fit in LDS
// (ceil(T/64) * E <= kGroupLdsCells): the bitmasks and per-chunk bases live in
// LDS, so the three steps need no round trips through memory and one launch.
// Outputs are identical to the three-kernel form.
constexpr int kGroupBatch = 16;

__global__ __launch_bounds__(1024) void k_group_fused(const int32_t* __restrict__ idx, int T, int k, int E,
                                                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm, int32_t* __restrict__ uniq,
                                                      int32_t* __restrict__ n_uniq) {
  __shared__ unsigned long long m[kGroupLdsCells];
  __shared__ int base[kGroupLdsCells];
  __shared__ int smem[64];
  const int tid = (int)threadIdx.x;
  const int C = (T + 63) / 64, cells = C * E, n = T * k;
  for (int i = tid; i < cells; i += 1024) m[i] = 0ull;
  __syncthreads();
  // assignments go kGroupBatch per thread at a time: their expert ids are all
  // requested before the first is used
  for (int f0 = 0; f0 < n; f0 += 1024 * kGroupBatch) {
    int ev[kGroupBatch];
#pragma unroll
    for (int j = 0; j < kGroupBatch; ++j) {
      const int f = f0 + 1024 * j + tid;
      ev[j] = f < n ? idx[f] : 0;
    }
#pragma unroll
    for (int j = 0; j < kGroupBatch; ++j) {
      const int f = f0 + 1024 * j + tid;
      if (f < n) {
        const int t = f / k;
        atomicOr(&m[(t >> 6) * E + ev[j]], 1ull << (t & 63));
      }
    }
  }
  __syncthreads();
  const int e = tid;
  int cnt = 0;
  if (e < E) {
    for (int c = 0; c < C; ++c) {
      base[c * E + e] = cnt;
      cnt += __popcll(m[c * E + e]);
    }
    counts[e] = cnt;
  }
  int total;
  const int off = block_exclusive_scan_1024(cnt, smem, total);
  if (e < E) {
    offsets[e] = off;
    for (int c = 0; c < C; ++c) base[c * E + e] += off;
  }
  if (e == 0) offsets[E] = total;
  int nu;
  const int pos = block_exclusive_scan_1024(cnt > 0 ? 1 : 0, smem, nu);
  if (e < E && cnt > 0) uniq[pos] = e;
  if (e == 0) *n_uniq = nu;
  __syncthreads();  // every expert's bases are in LDS
  for (int f0 = 0; f0 < n; f0 += 1024 * kGroupBatch) {
    int ev[kGroupBatch];
#pragma unroll
    for (int j = 0; j < kGroupBatch; ++j) {
      const int f = f0 + 1024 * j + tid;
      ev[j] = f < n ? idx[f] : 0;
    }
#pragma unroll
    for (int j = 0; j < kGroupBatch; ++j) {
      const int f = f0 + 1024 * j + tid;
      if (f < n) {
        const int t = f / k, cell = (t >> 6) * E + ev[j], bit = t & 63;
        const unsigned long long below = bit ? (m[cell] & ((1ull << bit) - 1ull)) : 0ull;
        perm[base[cell] + __popcll(below)] = f;
      }
    }
  }
}

// ---------------------------------------------------------------- launchers
// Router logits for batches on the matrix cores: v_mfma_f32_16x16x4_f32, fp32
// operands (activations upcast exactly) and fp32 accumulation, the precision of
// the router's gate linear ("QwenのMoEルーターを観測してホットエキスパートを先読みしても速くならなかった",
// section "ルーターをフックする").
// A workgroup owns a (16*MTT tokens) x (16*NTT experts) tile; its NW waves split
// its K range and add their partial tiles in LDS. Workgroups along blockIdx.z
// split K further and write separate partial planes, which the top-k adds. In the MFMA, lane l holds A[l%16][l/16],
// B[l/16][l%16] and D[4(l/16)+i][l%16]. A lane loads four consecutive K values
// of its token row and of its expert row at once and feeds one to each of four
// MFMAs: MFMA i of a step takes K values k + 4g + i (g = l/16), the same
// permutation on both operands, so the four MFMAs together cover k .. k+15.
typedef float float4v_r __attribute__((ext_vector_type(4)));
template <int XT, int MTT, int NTT>
__global__ __launch_bounds__(1024) void k_logits_mfma(const void* __restrict__ x, int T, int H,
                                                      const float* __restrict__ R, int E, float* __restrict__ logits,
                                                      int kw, int64_t ldr) {
  extern __shared__ float red[];  // [waves][MTT*NTT*4][64]
  // split blockIdx.z takes K range [z*nw*kw, (z+1)*nw*kw) into plane z
  logits += (int64_t)blockIdx.z * T * E;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * 16 * MTT, e0 = blockIdx.y * 16 * NTT;
  int64_t xrow[MTT];
  const float* rrow[NTT];
#pragma unroll
  for (int mt = 0; mt < MTT; ++mt) xrow[mt] = (int64_t)min(t0 + 16 * mt + r, T - 1) * H;
#pragma unroll
  for (int nt = 0; nt < NTT; ++nt) rrow[nt] = R + (int64_t)min(e0 + 16 * nt + r, E - 1) * ldr;
  float4v_r acc[MTT][NTT];
#pragma unroll
  for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTT; ++nt) acc[mt][nt] = float4v_r{0.f, 0.f, 0.f, 0.f};
  const int kb = (blockIdx.z * nw + w) * kw;
  for (int k = kb; k < kb + kw; k += 16) {
    float4 a[MTT], b[NTT];
#pragma unroll
    for (int mt = 0; mt < MTT; ++mt) a[mt] = load_x4<XT>(x, xrow[mt] + k + 4 * g);
#pragma unroll
    for (int nt = 0; nt < NTT; ++nt) b[nt] = *reinterpret_cast<const float4*>(rrow[nt] + k + 4 * g);
#pragma unroll
    for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTT; ++nt) {
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mt].x, b[nt].x, acc[mt][nt], 0, 0, 0);
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mt].y, b[nt].y, acc[mt][nt], 0, 0, 0);
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mt].z, b[nt].z, acc[mt][nt], 0, 0, 0);
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mt].w, b[nt].w, acc[mt][nt], 0, 0, 0);
      }
  }
  constexpr int NO = MTT * NTT * 4 * 64;  // outputs of the tile
  auto store = [&](int o, float v) {
    const int l = o & 63, i = (o >> 6) & 3, tile = o >> 8;
    const int mt = tile / NTT, nt = tile % NTT;
    const int t = t0 + 16 * mt + 4 * (l >> 4) + i, e = e0 + 16 * nt + (l & 15);
    if (t < T && e < E) logits[(int64_t)t * E + e] = v;
  };
  if (nw == 1) {
#pragma unroll
    for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) store(((mt * NTT + nt) * 4 + i) * 64 + lane, acc[mt][nt][i]);
    return;
  }
#pragma unroll
  for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w * NO + ((mt * NTT + nt) * 4 + i) * 64 + lane] = acc[mt][nt][i];
  __syncthreads();
  for (int o = threadIdx.x; o < NO; o += blockDim.x) {
    float v = 0.f;
    for (int j = 0; j < nw; ++j) v += red[j * NO + o];  // waves in K order
    store(o, v);
  }
}

// Router logits for bf16 activations on the bf16 matrix cores, at fp32 product
// accuracy. Each fp32 router weight is split exactly into three bf16 parts
// (hi: the top 8 significand bits, mid: the next 8 of the remainder, lo: the
// rest, at most 8 bits), so x * w = x * hi + x * mid + x * lo with every
// product exact; the MFMA adds them in fp32 like the fp32 kernel. The split is
// made in registers from the fp32 weights as they are loaded (4 bytes fetched
// per weight), and the products take three v_mfma_f32_16x16x32_bf16 per 32 K
// values instead of eight 16x16x4 fp32 MFMAs. Tiles, split-K planes and the
// output mapping are those of k_logits_mfma; lane (r = l%16, g = l/16) holds
// A[r][8g..8g+7] (a token row) and B[8g..8g+7][r] (an expert row), D[4g+i][r].
typedef __bf16 bf16x8_r __attribute__((ext_vector_type(8)));

template <typename F, int... Is>
__device__ __forceinline__ void router_static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
// f(0), ..., f(N-1) with compile-time indices
template <int N, typename F>
__device__ __forceinline__ void router_static_for(F&& f) {
  router_static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Token tiles (of 16) of the split-weight router kernel for large batches.
constexpr int kSplitTallM = 8;

// K steps of operands in flight per wave in k_logits_bf16x3: step i's MFMAs
// run while the loads of steps i+1 .. i+kRouterDepth-1 are outstanding.
constexpr int kRouterDepth = 3;

// The three bf16 parts of 8 fp32 weights, as MFMA operands: hi, mid, lo.
__device__ __forceinline__ void split_bf16x3(const float4v_r (&w)[2], bf16x8_r (&b)[3]) {
  uint32_t u[8], m[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = w[i >> 2][i & 3];
    u[i] = __builtin_bit_cast(uint32_t, v);
    const float r1 = v - __builtin_bit_cast(float, u[i] & 0xFFFF0000u);  // exact: the low 16 significand bits
    m[i] = __builtin_bit_cast(uint32_t, r1);
    const float r2 = r1 - __builtin_bit_cast(float, m[i] & 0xFFFF0000u);  // exact, at most 8 significant bits
    l[i] = __builtin_bit_cast(uint32_t, r2);
  }
  // element 2j in the low half of word j, 2j+1 in the high half: the top
  // halves of the two fp32 words
  typedef uint32_t u32x4_r __attribute__((ext_vector_type(4)));
  u32x4_r h4, m4, l4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h4[j] = __builtin_amdgcn_perm(u[2 * j + 1], u[2 * j], 0x07060302u);
    m4[j] = __builtin_amdgcn_perm(m[2 * j + 1], m[2 * j], 0x07060302u);
    l4[j] = __builtin_amdgcn_perm(l[2 * j + 1], l[2 * j], 0x07060302u);
  }
  b[0] = __builtin_bit_cast(bf16x8_r, h4);
  b[1] = __builtin_bit_cast(bf16x8_r, m4);
  b[2] = __builtin_bit_cast(bf16x8_r, l4);
}

template <int MTT, int NTT>
__global__ __launch_bounds__(256) void k_logits_bf16x3(const uint16_t* __restrict__ x, int T, int H,
                                                       const float* __restrict__ R, int64_t ldr, int E,
                                                       float* __restrict__ logits, int kw) {
  extern __shared__ float red[];  // [waves][MTT*NTT*4][64]
  logits += (int64_t)blockIdx.z * T * E;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * 16 * MTT, e0 = blockIdx.y * 16 * NTT;
  int64_t xrow[MTT], rrow[NTT];
#pragma unroll
  for (int mt = 0; mt < MTT; ++mt) xrow[mt] = (int64_t)min(t0 + 16 * mt + r, T - 1) * H;
#pragma unroll
  for (int nt = 0; nt < NTT; ++nt) rrow[nt] = (int64_t)min(e0 + 16 * nt + r, E - 1) * ldr;
  float4v_r acc[MTT][NTT];
#pragma unroll
  for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTT; ++nt) acc[mt][nt] = float4v_r{0.f, 0.f, 0.f, 0.f};
  const int kb = (blockIdx.z * nw + w) * kw;
  const int nsteps = kw / 32;
  // A ring of kRouterDepth register buffers, each one K step's fragments: the
  // loop is unrolled by the ring size so that every buffer index is a constant.
  bf16x8_r a[kRouterDepth][MTT];
  float4v_r wr[kRouterDepth][NTT][2];
  auto load = [&](auto S, int step) {
    constexpr int sl = decltype(S)::value;
    const int k = kb + 32 * step + 8 * g;
#pragma unroll
    for (int mt = 0; mt < MTT; ++mt) a[sl][mt] = *reinterpret_cast<const bf16x8_r*>(x + xrow[mt] + k);
#pragma unroll
    for (int nt = 0; nt < NTT; ++nt)
#pragma unroll
      for (int h = 0; h < 2; ++h) wr[sl][nt][h] = *reinterpret_cast<const float4v_r*>(R + rrow[nt] + k + 4 * h);
  };
  auto mma = [&](auto S) {
    constexpr int sl = decltype(S)::value;
#pragma unroll
    for (int nt = 0; nt < NTT; ++nt) {
      bf16x8_r b[3];
      split_bf16x3(wr[sl][nt], b);
#pragma unroll
      for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
        for (int p = 0; p < 3; ++p)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[sl][mt], b[p], acc[mt][nt], 0, 0, 0);
    }
  };
  router_static_for<kRouterDepth>([&](auto S) {
    if ((int)decltype(S)::value < nsteps) load(S, decltype(S)::value);
  });
  for (int i0 = 0; i0 < nsteps; i0 += kRouterDepth) {
    router_static_for<kRouterDepth>([&](auto S) {
      const int i = i0 + (int)decltype(S)::value;
      if (i < nsteps) {
        mma(S);
        if (i + kRouterDepth < nsteps) load(S, i + kRouterDepth);
      }
    });
  }
  constexpr int NO = MTT * NTT * 4 * 64;
  auto store = [&](int o, float v) {
    const int l = o & 63, i = (o >> 6) & 3, tile = o >> 8;
    const int mt = tile / NTT, nt = tile % NTT;
    const int t = t0 + 16 * mt + 4 * (l >> 4) + i, e = e0 + 16 * nt + (l & 15);
    if (t < T && e < E) logits[(int64_t)t * E + e] = v;
  };
  if (nw == 1) {
#pragma unroll
    for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) store(((mt * NTT + nt) * 4 + i) * 64 + lane, acc[mt][nt][i]);
    return;
  }
#pragma unroll
  for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w * NO + ((mt * NTT + nt) * 4 + i) * 64 + lane] = acc[mt][nt][i];
  __syncthreads();
  for (int o = threadIdx.x; o < NO; o += blockDim.x) {
    float v = 0.f;
    for (int j = 0; j < nw; ++j) v += red[j * NO + o];  // waves in K order
    store(o, v);
  }
}

// Waves per expert row in the few-token router kernel.
constexpr int kLogitsWaves = 4;

hipError_t launch_logits(const void* x, int xtype, int T, int H, const float* R, int E, float* logits,
                         int* nsplit, bool split_ok, hipStream_t s, int64_t ldr) {
  *nsplit = 1;
  if (ldr == 0) ldr = H;
  if (T >= kMfmaLogitsMinT) {
    // bf16 activations of a large batch: the split-weight bf16 kernel
    const bool split3 = xtype == MOE_BF16 && split_ok && T >= kSplitRouterMinT;
    const int kstep = split3 ? 32 : 16;
    // tile shape and split-K: aim for about two waves per SIMD (2048 waves)
    int mtt = T >= 32 && (int64_t)((T + 31) / 32) * ((E + 31) / 32) >= 128 ? 2 : 1;
    int ntt = E >= 32 && (int64_t)((T + 16 * mtt - 1) / (16 * mtt)) * ((E + 31) / 32) >= 128 ? 2 : 1;
    // The split-weight kernel is bound by what its tiles fetch from L2 (each
    // expert row in fp32, each token row in bf16): taller and wider tiles
    // fetch each row for more of the other side (mtt and ntt always name the
    // launched kernel's tile: the grid and the reduction's LDS follow them).
    if (split3 && ntt == 2 && (int64_t)((T + 16 * kSplitTallM - 1) / (16 * kSplitTallM)) * ((E + 31) / 32) >= 128) {
      mtt = kSplitTallM;
      // wider expert tiles once there are enough of them
      if ((int64_t)((T + 16 * kSplitTallM - 1) / (16 * kSplitTallM)) * ((E + 63) / 64) >= 256) ntt = 4;
    }
    dim3 grid((T + 16 * mtt - 1) / (16 * mtt), (E + 16 * ntt - 1) / (16 * ntt));
    const int64_t tiles = (int64_t)grid.x * grid.y;
    // waves per workgroup (up to 4), then K splits across workgroups, while the
    // total stays within about 2048 waves and every wave keeps >= 64 of K
    int nw = 1, ns = 1;
    auto fits = [&](int w, int sp) {
      return tiles * w * sp <= 2048 && H % (kstep * w * sp) == 0 && H / (w * sp) >= 64;
    };
    while (nw < 4 && fits(nw * 2, ns)) nw *= 2;
    while (ns < logits_max_splits(T, E) && fits(nw, ns * 2)) ns *= 2;
    grid.z = ns;
    *nsplit = ns;
    const int kw = H / (nw * ns);
    const size_t lds = nw > 1 ? (size_t)nw * mtt * ntt * 256 * sizeof(float) : 0;
    auto go = [&](auto XC, auto MC, auto NC) {
      constexpr int X_ = decltype(XC)::value, M_ = decltype(MC)::value, N_ = decltype(NC)::value;
      if (split3)
        MOE_LAUNCH(MOE_KERNEL_ROUTE_LOGITS, (k_logits_bf16x3<M_, N_>), grid, dim3(64 * nw), lds, s,
                   static_cast<const uint16_t*>(x), T, H, R, ldr, E, logits, kw);
      else
        MOE_LAUNCH(MOE_KERNEL_ROUTE_LOGITS, (k_logits_mfma<X_, M_, N_>), grid, dim3(64 * nw), lds, s, x, T, H, R, E,
                   logits, kw, ldr);
    };
    auto with_tile = [&](auto XC) {
      if (mtt == kSplitTallM) {
        if (ntt == 4)
          MOE_LAUNCH(MOE_KERNEL_ROUTE_LOGITS, (k_logits_bf16x3<kSplitTallM, 4>), grid, dim3(64 * nw), lds, s,
                     static_cast<const uint16_t*>(x), T, H, R, ldr, E, logits, kw);
        else
          MOE_LAUNCH(MOE_KERNEL_ROUTE_LOGITS, (k_logits_bf16x3<kSplitTallM, 2>), grid, dim3(64 * nw), lds, s,
                     static_cast<const uint16_t*>(x), T, H, R, ldr, E, logits, kw);
        return;
      }
      if (mtt == 2 && ntt == 2) go(XC, std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{});
      else if (ntt == 2) go(XC, std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{});
      else if (mtt == 2) go(XC, std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{});
      else go(XC, std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
    };
    switch (xtype) {
      case MOE_F32: with_tile(std::integral_constant<int, MOE_F32>{}); break;
      case MOE_F16: with_tile(std::integral_constant<int, MOE_F16>{}); break;
      default: with_tile(std::integral_constant<int, MOE_BF16>{}); break;
    }
  } else {
    // chunks of 256 columns per wave, kLogitsWaves waves per expert row
    const int nch = ((H + 255) / 256 + kLogitsWaves - 1) / kLogitsWaves;
    auto go = [&](auto NC) {
      constexpr int N = decltype(NC)::value, WPE = kLogitsWaves;
      constexpr int TU = N >= 16 ? 2 : N >= 8 ? 4 : 8;
      const dim3 block(64 * WPE);
      // a single token takes the one-token unroll (no repeated activation loads)
      auto launch = [&](auto TUc) {
        constexpr int U = decltype(TUc)::value;
        switch (xtype) {
          case MOE_F32: MOE_LAUNCH(MOE_KERNEL_ROUTE_LOGITS, (k_logits_rows<MOE_F32, N, U, WPE>), dim3(E), block, 0, s, x, T, H, R, E, logits); break;
          case MOE_F16: MOE_LAUNCH(MOE_KERNEL_ROUTE_LOGITS, (k_logits_rows<MOE_F16, N, U, WPE>), dim3(E), block, 0, s, x, T, H, R, E, logits); break;
          default:      MOE_LAUNCH(MOE_KERNEL_ROUTE_LOGITS, (k_logits_rows<MOE_BF16, N, U, WPE>), dim3(E), block, 0, s, x, T, H, R, E, logits); break;
        }
      };
      if (T == 1) launch(std::integral_constant<int, 1>{});
      else launch(std::integral_constant<int, TU>{});
    };
    if (nch <= 1) go(std::integral_constant<int, 1>{});
    else if (nch <= 2) go(std::integral_constant<int, 2>{});
    else if (nch <= 4) go(std::integral_constant<int, 4>{});
    else if (nch <= 8) go(std::integral_constant<int, 8>{});
    else go(std::integral_constant<int, 16>{});
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int nsplit, int T, int E, int k, int renorm, int32_t* idx, float* gate,
                       int32_t* idx2, float* gate2, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  const int vpl = (E + 63) / 64;
  if (vpl <= 1)      MOE_LAUNCH(MOE_KERNEL_TOPK, k_topk<1>, grid, dim3(256), 0, s, logits, nsplit, T, E, k, renorm, idx, gate, idx2, gate2);
  else if (vpl <= 2) MOE_LAUNCH(MOE_KERNEL_TOPK, k_topk<2>, grid, dim3(256), 0, s, logits, nsplit, T, E, k, renorm, idx, gate, idx2, gate2);
  else if (vpl <= 4) MOE_LAUNCH(MOE_KERNEL_TOPK, k_topk<4>, grid, dim3(256), 0, s, logits, nsplit, T, E, k, renorm, idx, gate, idx2, gate2);
  else if (vpl <= 8) MOE_LAUNCH(MOE_KERNEL_TOPK, k_topk<8>, grid, dim3(256), 0, s, logits, nsplit, T, E, k, renorm, idx, gate, idx2, gate2);
  else               MOE_LAUNCH(MOE_KERNEL_TOPK, k_topk<16>, grid, dim3(256), 0, s, logits, nsplit, T, E, k, renorm, idx, gate, idx2, gate2);
  return hipGetLastError();
}

hipError_t launch_group(const int32_t* idx, int T, int k, int E, const GroupBufs& g, hipStream_t s) {
  const int C = (T + 63) / 64;
  if ((int64_t)C * E <= kGroupLdsCells) {
    MOE_LAUNCH(MOE_KERNEL_GROUP, k_group_fused, dim3(1), dim3(1024), 0, s, idx, T, k, E, g.counts, g.offsets, g.perm,
               g.uniq, g.n_uniq);
    return hipGetLastError();
  }
  MOE_LAUNCH(MOE_KERNEL_GROUP, k_group_mask, dim3(C), dim3(256), 0, s, idx, T, k, E, g.mask);
  MOE_LAUNCH(MOE_KERNEL_GROUP, k_group_scan, dim3(1), dim3(1024), 0, s, g.mask, C, E, g.base, g.counts, g.offsets, g.uniq,
                     g.n_uniq);
  const int64_t n = (int64_t)T * k;
  MOE_LAUNCH(MOE_KERNEL_GROUP, k_group_scatter, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, idx, T, k, E, g.mask,
                     g.base, g.perm);
  return hipGetLastError();
}

}  // namespace moe

MOE_STAMP_READER(moe_stamps_read_route, moe::g_stamps_route);
#ifdef MOE_STAMPS
// frequency of the stamps' counter on the current device, in kHz (0 on error)
extern "C" int moe_stamps_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return 0;
  return khz;
}
#endif
