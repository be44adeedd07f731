// k_decode.hip — gathered block-quantized expert kernels for decode (matvec shape).
//
// [QK] "鳴かぬなら、カスタムカーネル、ほととぎす" (qiita.com, john-rocky):
//   section 4: the routed expert id is a kernel input that indexes the weight
//   reads, so the other experts' weights are never fetched;
//   section 6: codes are symmetric linear int8 with a scale per 32 K elements;
//   section 7: gate and up share the token; the down projection of each slot
//   takes that expert's own gated activation.
// [LR] "QwenのMoEルーターを観測してホットエキスパートを先読みしても速くならなかった"
//   section "事前ウォームアップとmmapキャッシュを比べる": the experts are one stacked
//   (experts, out, in) array and gather_qmm picks rows by expert index.
//
// Lane mapping: a lane owns whole quantisation blocks (32 codes, one scale), so
// each code row is read with coalesced 16-byte loads, dequantised in registers
// and the scale applied once per block partial.
#include <type_traits>

#include "kernels.hpp"

namespace moe {

template <int V>
using IC = std::integral_constant<int, V>;

template <typename F>
static void with_scheme(int scheme, F&& f) {
  if (scheme == MOE_Q_SYM8) f(IC<MOE_Q_SYM8>{});
  else f(IC<MOE_Q_INT4>{});
}

template <typename F>
static void with_xtype(int xt, F&& f) {
  if (xt == MOE_F32) f(IC<MOE_F32>{});
  else if (xt == MOE_F16) f(IC<MOE_F16>{});
  else f(IC<MOE_BF16>{});
}

template <int SCHEME>
__host__ __device__ constexpr int64_t row_bytes(int K) {
  return SCHEME == MOE_Q_SYM8 ? (int64_t)K : (int64_t)K / 2;
}

// ------------------------------------------------------------------ T = 1
// Grid: k slots x blocks_per_slot. A wave computes RP (gate row n, up row I+n)
// pairs of its slot's expert and writes h[slot][n] = silu(gate) * up.
// With FROM_LOGITS the wave first picks the top k from the router logits (each
// workgroup redoes this small step so no cross-workgroup sync is needed);
// workgroup 0 publishes the routing for the down kernel and the caller.
template <int SCHEME, int XT, int NBJ, int RP, bool FROM_LOGITS, int VPL>
__global__ __launch_bounds__(256) void k_gate_up_t1(const void* __restrict__ x, ExpertsDev ex, int k, int renorm,
                                                    const float* __restrict__ logits,
                                                    const int32_t* __restrict__ idx_in,
                                                    int32_t* __restrict__ idx_ws, float* __restrict__ gate_ws,
                                                    int32_t* __restrict__ idx_user, float* __restrict__ gate_user,
                                                    float* __restrict__ h, int blocks_per_slot) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slot = blockIdx.x / blocks_per_slot, blk = blockIdx.x % blocks_per_slot;
  int e;
  if constexpr (FROM_LOGITS) {
    int my_idx;
    float my_gate;
    wave_topk<VPL>(logits, ex.E, k, renorm != 0, my_idx, my_gate);
    if (blockIdx.x == 0 && wave == 0 && lane < k) {
      idx_ws[lane] = my_idx;
      gate_ws[lane] = my_gate;
      if (idx_user) idx_user[lane] = my_idx;
      if (gate_user) gate_user[lane] = my_gate;
    }
    e = __shfl(my_idx, slot, 64);
  } else {
    e = idx_in[slot];
  }
  const int H = ex.H, I = ex.I, NB = H / 32;
  float xf[NBJ][32];
#pragma unroll
  for (int j = 0; j < NBJ; ++j) {
    const int b = lane + 64 * j;
    if (b < NB) load_x_block<XT>(x, 0, b, xf[j]);
    else {
#pragma unroll
      for (int i = 0; i < 32; ++i) xf[j][i] = 0.0f;
    }
  }
  const int n0 = (blk * 4 + wave) * RP;
  const int64_t rb = row_bytes<SCHEME>(H);
  Block<SCHEME> cg[RP][NBJ], cu[RP][NBJ];
  float sg[RP][NBJ], su[RP][NBJ];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int n = min(n0 + r, I - 1);  // rows past I are read in bounds and discarded
    const int64_t grow = (int64_t)e * 2 * I + n, urow = grow + I;
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      const int b = lane + 64 * j;
      if (b < NB) {
        cg[r][j] = load_block<SCHEME>(ex.wgu + grow * rb, b);
        cu[r][j] = load_block<SCHEME>(ex.wgu + urow * rb, b);
        sg[r][j] = f16_bits_to_f32(ex.sgu[grow * NB + b]);
        su[r][j] = f16_bits_to_f32(ex.sgu[urow * NB + b]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    float ag = 0.0f, au = 0.0f;
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      if (lane + 64 * j < NB) {
        ag = fmaf(sg[r][j], block_dot<SCHEME>(cg[r][j], xf[j]), ag);
        au = fmaf(su[r][j], block_dot<SCHEME>(cu[r][j], xf[j]), au);
      }
    }
    ag = wave_sum(ag);
    au = wave_sum(au);
    if (lane == 0 && n0 + r < I) h[(int64_t)slot * I + n0 + r] = silu(ag) * au;
  }
}

// Grid: ceil(H / 16). 16 lanes per output row, 4 rows per wave. For each slot in
// order: row of the slot's expert . h[slot], then y += gate * that (or, with
// gate == nullptr, y[slot][m] = that).
template <int SCHEME, int NBJ>
__global__ __launch_bounds__(256) void k_down_t1(ExpertsDev ex, int k, const int32_t* __restrict__ idx,
                                                 const float* __restrict__ gate, const float* __restrict__ h,
                                                 float* __restrict__ y) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lg = lane >> 4, ll = lane & 15;
  const int H = ex.H, I = ex.I, NBI = I / 32;
  const int m = (blockIdx.x * 4 + wave) * 4 + lg;
  const int mm = min(m, H - 1);
  const int64_t rb = row_bytes<SCHEME>(I);
  float acc = 0.0f;
#pragma unroll 2
  for (int s = 0; s < k; ++s) {
    const int e = idx[s];
    const int64_t row = (int64_t)e * H + mm;
    Block<SCHEME> c[NBJ];
    float sc[NBJ];
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      const int b = ll + 16 * j;
      if (b < NBI) {
        c[j] = load_block<SCHEME>(ex.wd + row * rb, b);
        sc[j] = f16_bits_to_f32(ex.sd[row * NBI + b]);
      }
    }
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      const int b = ll + 16 * j;
      if (b < NBI) {
        float hv[32];
        const float4* hp = reinterpret_cast<const float4*>(h + (int64_t)s * I + 32 * b);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 v = hp[i];
          hv[4 * i] = v.x; hv[4 * i + 1] = v.y; hv[4 * i + 2] = v.z; hv[4 * i + 3] = v.w;
        }
        part = fmaf(sc[j], block_dot<SCHEME>(c[j], hv), part);
      }
    }
    part = group_sum<16>(part);
    if (gate) acc = fmaf(gate[s], part, acc);
    else if (ll == 0 && m < H) y[(int64_t)s * H + m] = part;
  }
  if (gate && ll == 0 && m < H) y[m] = acc;
}

// ------------------------------------------------------------------ T > 1, grouped
// Grid: (blocks_per_u, max unique experts). Workgroup column u serves expert
// uniq[u] for all of its n_e assignments: the code rows are loaded once and
// dotted with each routed token, so a batch reads each routed expert once.
template <int SCHEME, int XT, int NBJ, int RP>
__global__ __launch_bounds__(256) void k_gate_up_grouped(const void* __restrict__ x, ExpertsDev ex, int k,
                                                         const int32_t* __restrict__ uniq,
                                                         const int32_t* __restrict__ n_uniq,
                                                         const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ perm, float* __restrict__ h) {
  const int u = blockIdx.y;
  if (u >= *n_uniq) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = uniq[u], cnt = counts[e], beg = offsets[e];
  const int H = ex.H, I = ex.I, NB = H / 32;
  const int n0 = (blockIdx.x * 4 + wave) * RP;
  const int64_t rb = row_bytes<SCHEME>(H);
  Block<SCHEME> cg[RP][NBJ], cu[RP][NBJ];
  float sg[RP][NBJ], su[RP][NBJ];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int n = min(n0 + r, I - 1);
    const int64_t grow = (int64_t)e * 2 * I + n, urow = grow + I;
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      const int b = lane + 64 * j;
      if (b < NB) {
        cg[r][j] = load_block<SCHEME>(ex.wgu + grow * rb, b);
        cu[r][j] = load_block<SCHEME>(ex.wgu + urow * rb, b);
        sg[r][j] = f16_bits_to_f32(ex.sgu[grow * NB + b]);
        su[r][j] = f16_bits_to_f32(ex.sgu[urow * NB + b]);
      }
    }
  }
  for (int a = 0; a < cnt; ++a) {
    const int f = perm[beg + a];
    const int t = f / k;
    float ag[RP], au[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) ag[r] = au[r] = 0.0f;
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      const int b = lane + 64 * j;
      if (b < NB) {
        float xf[32];
        load_x_block<XT>(x, (int64_t)t * H, b, xf);
#pragma unroll
        for (int r = 0; r < RP; ++r) {
          ag[r] = fmaf(sg[r][j], block_dot<SCHEME>(cg[r][j], xf), ag[r]);
          au[r] = fmaf(su[r][j], block_dot<SCHEME>(cu[r][j], xf), au[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const float g = wave_sum(ag[r]);
      const float v = wave_sum(au[r]);
      if (lane == 0 && n0 + r < I) h[(int64_t)f * I + n0 + r] = silu(g) * v;
    }
  }
}

// Grid: (ceil(H / 16), max unique experts). ys[f][m] = row m of expert uniq[u] . h[f]
// for each assignment f of that expert.
template <int SCHEME, int NBJ>
__global__ __launch_bounds__(256) void k_down_grouped(ExpertsDev ex, int k, const int32_t* __restrict__ uniq,
                                                      const int32_t* __restrict__ n_uniq,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ perm, const float* __restrict__ h,
                                                      float* __restrict__ ys) {
  const int u = blockIdx.y;
  if (u >= *n_uniq) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lg = lane >> 4, ll = lane & 15;
  const int e = uniq[u], cnt = counts[e], beg = offsets[e];
  const int H = ex.H, I = ex.I, NBI = I / 32;
  const int m = (blockIdx.x * 4 + wave) * 4 + lg;
  const int mm = min(m, H - 1);
  const int64_t rb = row_bytes<SCHEME>(I);
  const int64_t row = (int64_t)e * H + mm;
  Block<SCHEME> c[NBJ];
  float sc[NBJ];
#pragma unroll
  for (int j = 0; j < NBJ; ++j) {
    const int b = ll + 16 * j;
    if (b < NBI) {
      c[j] = load_block<SCHEME>(ex.wd + row * rb, b);
      sc[j] = f16_bits_to_f32(ex.sd[row * NBI + b]);
    }
  }
  for (int a = 0; a < cnt; ++a) {
    const int f = perm[beg + a];
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      const int b = ll + 16 * j;
      if (b < NBI) {
        float hv[32];
        const float4* hp = reinterpret_cast<const float4*>(h + (int64_t)f * I + 32 * b);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 v = hp[i];
          hv[4 * i] = v.x; hv[4 * i + 1] = v.y; hv[4 * i + 2] = v.z; hv[4 * i + 3] = v.w;
        }
        part = fmaf(sc[j], block_dot<SCHEME>(c[j], hv), part);
      }
    }
    part = group_sum<16>(part);
    if (ll == 0 && m < H) ys[(int64_t)f * H + m] = part;
  }
}

// y[t][m] = sum over slots s, in order, of gate[t][s] * ys[t*k+s][m].
__global__ __launch_bounds__(256) void k_combine(int T, int H, int k, const float* __restrict__ gate,
                                                 const float* __restrict__ ys, float* __restrict__ y) {
  const int nbx = (H + 255) / 256;
  const int t = blockIdx.x / nbx;
  const int m = (blockIdx.x % nbx) * 256 + threadIdx.x;
  if (t >= T || m >= H) return;
  float acc = 0.0f;
  for (int s = 0; s < k; ++s) acc = fmaf(gate[(int64_t)t * k + s], ys[((int64_t)t * k + s) * H + m], acc);
  y[(int64_t)t * H + m] = acc;
}

// ------------------------------------------------------------------ launchers
hipError_t launch_decode_t1(const void* x, int xtype, const ExpertsDev& ex, int k, int renorm,
                            const float* logits, const int32_t* idx_in, const float* gate_in,
                            int32_t* idx_ws, float* gate_ws, int32_t* idx_user, float* gate_user,
                            float* h, float* y, hipStream_t s) {
  const bool from_logits = logits != nullptr;
  const int nbj = (ex.H / 32 + 63) / 64;  // 1 (H <= 2048) or 2 (H <= 4096)
  with_scheme(ex.scheme, [&](auto S) {
    with_xtype(xtype, [&](auto X) {
      constexpr int SC = decltype(S)::value, XT = decltype(X)::value;
      auto go = [&](auto NBJc, auto RPc) {
        constexpr int NBJ = decltype(NBJc)::value, RP = decltype(RPc)::value;
        const int bps = (ex.I + 4 * RP - 1) / (4 * RP);
        dim3 grid(k * bps);
        if (!from_logits)
          hipLaunchKernelGGL((k_gate_up_t1<SC, XT, NBJ, RP, false, 1>), grid, dim3(256), 0, s, x, ex, k, renorm,
                             logits, idx_in, idx_ws, gate_ws, idx_user, gate_user, h, bps);
        else if (ex.E <= 256)
          hipLaunchKernelGGL((k_gate_up_t1<SC, XT, NBJ, RP, true, 4>), grid, dim3(256), 0, s, x, ex, k, renorm,
                             logits, idx_in, idx_ws, gate_ws, idx_user, gate_user, h, bps);
        else
          hipLaunchKernelGGL((k_gate_up_t1<SC, XT, NBJ, RP, true, 16>), grid, dim3(256), 0, s, x, ex, k, renorm,
                             logits, idx_in, idx_ws, gate_ws, idx_user, gate_user, h, bps);
      };
      if (nbj <= 1) go(IC<1>{}, IC<4>{});
      else go(IC<2>{}, IC<2>{});
    });
  });
  const int32_t* idx = from_logits ? idx_ws : idx_in;
  const float* gate = from_logits ? gate_ws : gate_in;
  const int nbi = (ex.I / 32 + 15) / 16;
  dim3 grid((ex.H + 15) / 16);
  with_scheme(ex.scheme, [&](auto S) {
    constexpr int SC = decltype(S)::value;
    if (nbi <= 1) hipLaunchKernelGGL((k_down_t1<SC, 1>), grid, dim3(256), 0, s, ex, k, idx, gate, h, y);
    else if (nbi <= 2) hipLaunchKernelGGL((k_down_t1<SC, 2>), grid, dim3(256), 0, s, ex, k, idx, gate, h, y);
    else if (nbi <= 4) hipLaunchKernelGGL((k_down_t1<SC, 4>), grid, dim3(256), 0, s, ex, k, idx, gate, h, y);
    else hipLaunchKernelGGL((k_down_t1<SC, 8>), grid, dim3(256), 0, s, ex, k, idx, gate, h, y);
  });
  return hipGetLastError();
}

hipError_t launch_decode_grouped(const void* x, int xtype, int T, const ExpertsDev& ex, int k,
                                 const GroupBufs& g, const float* gate, float* h, float* ys, float* y,
                                 hipStream_t s) {
  const int maxu = (int)std::min<int64_t>((int64_t)ex.E, (int64_t)T * k);
  const int nbj = (ex.H / 32 + 63) / 64;
  with_scheme(ex.scheme, [&](auto S) {
    with_xtype(xtype, [&](auto X) {
      constexpr int SC = decltype(S)::value, XT = decltype(X)::value;
      auto go = [&](auto NBJc, auto RPc) {
        constexpr int NBJ = decltype(NBJc)::value, RP = decltype(RPc)::value;
        dim3 grid((ex.I + 4 * RP - 1) / (4 * RP), maxu);
        hipLaunchKernelGGL((k_gate_up_grouped<SC, XT, NBJ, RP>), grid, dim3(256), 0, s, x, ex, k, g.uniq, g.n_uniq,
                           g.counts, g.offsets, g.perm, h);
      };
      if (nbj <= 1) go(IC<1>{}, IC<4>{});
      else go(IC<2>{}, IC<2>{});
    });
  });
  float* out = gate ? ys : y;  // per-slot mode writes [T][k][H] directly
  const int nbi = (ex.I / 32 + 15) / 16;
  dim3 grid((ex.H + 15) / 16, maxu);
  with_scheme(ex.scheme, [&](auto S) {
    constexpr int SC = decltype(S)::value;
    if (nbi <= 1) hipLaunchKernelGGL((k_down_grouped<SC, 1>), grid, dim3(256), 0, s, ex, k, g.uniq, g.n_uniq, g.counts, g.offsets, g.perm, h, out);
    else if (nbi <= 2) hipLaunchKernelGGL((k_down_grouped<SC, 2>), grid, dim3(256), 0, s, ex, k, g.uniq, g.n_uniq, g.counts, g.offsets, g.perm, h, out);
    else if (nbi <= 4) hipLaunchKernelGGL((k_down_grouped<SC, 4>), grid, dim3(256), 0, s, ex, k, g.uniq, g.n_uniq, g.counts, g.offsets, g.perm, h, out);
    else hipLaunchKernelGGL((k_down_grouped<SC, 8>), grid, dim3(256), 0, s, ex, k, g.uniq, g.n_uniq, g.counts, g.offsets, g.perm, h, out);
  });
  if (gate) {
    dim3 cg((unsigned)(((ex.H + 255) / 256) * (int64_t)T));
    hipLaunchKernelGGL(k_combine, cg, dim3(256), 0, s, T, ex.H, k, gate, ys, y);
  }
  return hipGetLastError();
}

}  // namespace moe
