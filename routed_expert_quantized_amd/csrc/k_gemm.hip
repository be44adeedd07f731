// k_gemm.hip — grouped MFMA GEMM for batched tokens (prefill and batched decode).
//
// After the token-by-expert grouping each routed expert e has n_e assignments.
// GEMM1: U_e[n_e][2I] = X_e[n_e][H] . W_gu[e]^T, then h = silu(gate) * up
//        (gate columns n and up columns I + n in the same workgroup), stored fp16.
// GEMM2: Y_e[n_e][H] = h_e[n_e][I] . W_d[e]^T, stored fp32 per assignment (ys).
// Each expert's weights are read once per pass over its assignments
// ("鳴かぬなら、カスタムカーネル、ほととぎす", section 4: only routed experts are read;
// section 7: each slot's down projection takes that slot's own activation).
//
// Arithmetic: v_mfma_f32_16x16x32_f16 with fp32 accumulation. Weights are
// dequantised in registers as fp16(code * scale), one rounding (codes and
// scales are exact in fp16); activations are staged as fp16 (exact for fp16
// input, one rounding for bf16 values below the fp16 normal range or for fp32).
//
// Operand layout of the MFMA (checked on gfx950): lane l holds A[l%16][8(l/16)+j],
// B[8(l/16)+j][l%16] for j < 8, and D[4(l/16)+i][l%16] for i < 4. A K chunk
// covers one 128-byte line of every weight row: four sym8 blocks (K=128) or
// eight int4 blocks (K=256). Lane group g = l/16 loads BPG = 1 (sym8) or 2
// (int4) whole consecutive blocks of its row, so the four groups read the line
// together and no half line is left for a later refetch; MFMA j of the chunk
// takes elements 8(j%4)..8(j%4)+7 of the group's block j/4, which is chunk
// element 32*BPG*g + 8j. The A tile in LDS is laid out to match (for int4 the
// pair order of the nibble unpacking is mirrored in A while staging). Since
// the scale is folded into B, mixing blocks across lane groups inside one MFMA
// is exact.
#include <algorithm>
#include <type_traits>

#include "kernels.hpp"

namespace moe {

typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

template <int V>
using ICg = std::integral_constant<int, V>;

// blocks per lane group and K per chunk (one 128-byte weight line per row)
template <int SCHEME>
constexpr int gemm_bpg() { return SCHEME == MOE_Q_INT4 ? 2 : 1; }
template <int SCHEME>
constexpr int gemm_kc() { return 128 * gemm_bpg<SCHEME>(); }
template <int SCHEME>
constexpr int gemm_arow() { return gemm_kc<SCHEME>() * 2 + 16; }  // bytes per LDS A row (fp16 + pad)

// 8 fp16 values: elements 8j..8j+7 of a 32-code block, times the block scale.
template <int SCHEME>
__device__ __forceinline__ half8v block_slice_f16(const Block<SCHEME>& blk, int j, half2v s2) {
  half8v r;
  if constexpr (SCHEME == MOE_Q_SYM8) {
    const half2v bias = as_h2(0xE480E480u);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t u = blk.w[2 * j + w] ^ 0x80808080u;
      const half2v lo = (as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) + bias) * s2;
      const half2v hi = (as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) + bias) * s2;
      r[4 * w + 0] = lo[0]; r[4 * w + 1] = lo[1]; r[4 * w + 2] = hi[0]; r[4 * w + 3] = hi[1];
    }
  } else {
    // codes 8j..8j+7 are word j; pairs come out as (c0,c4),(c1,c5),(c2,c6),(c3,c7)
    const half2v bias = as_h2(0xE408E408u);
    const uint32_t u = blk.w[j] ^ 0x88888888u;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const half2v v = (as_h2(((u >> (4 * p)) & 0x000F000Fu) | 0x64006400u) + bias) * s2;
      r[2 * p] = v[0];
      r[2 * p + 1] = v[1];
    }
  }
  return r;
}

// Converts 8 source activations (natural order) to the fp16 order B uses.
template <int SCHEME>
__device__ __forceinline__ uint4 order_for_b(uint4 h) {
  if constexpr (SCHEME == MOE_Q_SYM8) {
    return h;
  } else {
    // natural pairs (x0,x1)(x2,x3)(x4,x5)(x6,x7) -> (x0,x4)(x1,x5)(x2,x6)(x3,x7)
    uint4 r;
    r.x = __builtin_amdgcn_perm(h.z, h.x, 0x05040100u);
    r.y = __builtin_amdgcn_perm(h.z, h.x, 0x07060302u);
    r.z = __builtin_amdgcn_perm(h.w, h.y, 0x05040100u);
    r.w = __builtin_amdgcn_perm(h.w, h.y, 0x07060302u);
    return r;
  }
}

// 8 activations starting at element i of a row, as packed fp16 (natural order).
template <int XT>
__device__ __forceinline__ uint4 load8_f16(const uint8_t* row, int i) {
  if constexpr (XT == MOE_F16) {
    return *reinterpret_cast<const uint4*>(row + 2 * i);
  } else if constexpr (XT == MOE_BF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + 2 * i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const half2v hp = {(_Float16)bf16_bits_to_f32((uint16_t)(w[q] & 0xFFFF)),
                         (_Float16)bf16_bits_to_f32((uint16_t)(w[q] >> 16))};
      o[q] = __builtin_bit_cast(uint32_t, hp);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(row + 4 * i);
    const float4 b = *reinterpret_cast<const float4*>(row + 4 * i + 16);
    const half2v p0 = {(_Float16)a.x, (_Float16)a.y}, p1 = {(_Float16)a.z, (_Float16)a.w};
    const half2v p2 = {(_Float16)b.x, (_Float16)b.y}, p3 = {(_Float16)b.z, (_Float16)b.w};
    return make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                      __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
  }
}

// Grid: (column blocks per expert, max unique experts); 256 threads, 4 waves.
// MODE 0 (gate/up): wave w owns gate rows n0+16w.. and up rows I+n0+16w.., a
//   workgroup owns 64 gate/up pairs; output h16[f][n] = fp16(silu(g) * u).
// MODE 1 (down): wave w owns rows n0+32w .. n0+32w+31 of W_d[e]; a workgroup
//   owns 128 rows; output ys[f][n] (fp32).
// The expert's assignments are taken 16*MT at a time (one pass each).
template <int SCHEME, int XT, int MODE, int MT>
__global__ __launch_bounds__(256) void k_gemm_grouped(const void* __restrict__ act, ExpertsDev ex, int k,
                                                      const int32_t* __restrict__ uniq,
                                                      const int32_t* __restrict__ n_uniq,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ perm, uint16_t* __restrict__ h16,
                                                      float* __restrict__ ys) {
  constexpr int BPG = gemm_bpg<SCHEME>(), KC = gemm_kc<SCHEME>(), AROW = gemm_arow<SCHEME>();
  constexpr int NJ = KC / 32;  // MFMAs per chunk per output tile
  __shared__ __attribute__((aligned(16))) uint8_t As[16 * MT * AROW];
  __shared__ int fs[16 * MT];
  const int u = blockIdx.y;
  if (u >= *n_uniq) return;
  const int tid = (int)threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, r16 = lane & 15;
  const int e = uniq[u], cnt = counts[e], beg = offsets[e];
  const int H = ex.H, I = ex.I;
  const int K = MODE == 0 ? H : I;          // reduction length
  const int NB = K / 32;                    // quantisation blocks per weight row
  const int NROW = MODE == 0 ? 2 * I : H;   // weight rows of this expert
  const int lim = MODE == 0 ? I : H;        // valid output columns
  const uint8_t* W = MODE == 0 ? ex.wgu : ex.wd;
  const uint16_t* S = MODE == 0 ? ex.sgu : ex.sd;
  const int64_t rb = row_bytes<SCHEME>(K);
  constexpr int xbytes = MODE == 1 ? 2 : (XT == MOE_F32 ? 4 : 2);
  const int64_t arow_bytes = (int64_t)K * xbytes;
  const uint8_t* Ab = static_cast<const uint8_t*>(act);

  // this wave's two 16-row column tiles
  int col[2];
  if (MODE == 0) {
    const int n0 = blockIdx.x * 64 + wave * 16;
    col[0] = n0;       // gate
    col[1] = I + n0;   // up
  } else {
    const int n0 = blockIdx.x * 128 + wave * 32;
    col[0] = n0;
    col[1] = n0 + 16;
  }
  int64_t wrow[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int rr = min(col[c] + r16, NROW - 1);
    wrow[c] = (int64_t)e * NROW + rr;
  }
  const int nchunks = (NB + 4 * BPG - 1) / (4 * BPG);

  for (int m0 = 0; m0 < cnt; m0 += 16 * MT) {
    const int nm = min(16 * MT, cnt - m0);
    __syncthreads();
    if (tid < 16 * MT) fs[tid] = tid < nm ? perm[beg + m0 + tid] : -1;
    __syncthreads();
    float4v acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[mt][c] = float4v{0.f, 0.f, 0.f, 0.f};

    constexpr int PPR = KC / 8;                 // 16-byte activation pieces per row per chunk
    constexpr int NST = 16 * MT * PPR / 256;    // pieces per thread per chunk
    static_assert((16 * MT * PPR) % 256 == 0, "activation tile must split evenly over 256 threads");
    const int mtiles = (nm + 15) / 16;          // M tiles holding assignments (uniform)
    // Thread tid stages pieces c = tid + 256 i: row c / PPR, column group tid % PPR
    // (256 is a multiple of PPR). The rows' source offsets are fixed for the pass,
    // so they are found once here (rows past the assignments repeat row 0).
    const int grp8 = (tid % PPR) * 8;
    uint32_t aoff[NST];
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int row = tid / PPR + i * (256 / PPR);
      const int f = fs[row] >= 0 ? fs[row] : fs[0];
      const uint32_t src = MODE == 0 ? (uint32_t)(f / k) : (uint32_t)f;
      aoff[i] = src * (uint32_t)arow_bytes;
    }
    // chunk loads: lane group g holds blocks 4*BPG*q + BPG*g + b (b < BPG) of
    // its weight rows; the activation tile is 16*MT rows x KC elements, 8
    // elements per piece
    auto load_w = [&](int q, Block<SCHEME> (*wb)[BPG], half2v (*s2)[BPG]) {
#pragma unroll
      for (int b = 0; b < BPG; ++b) {
        const int blk = 4 * BPG * q + BPG * g + b;
        const int bc = min(blk, NB - 1);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          wb[c][b] = load_block<SCHEME>(W + wrow[c] * rb, bc);
          const float sv = blk < NB ? f16_bits_to_f32(S[wrow[c] * NB + bc]) : 0.0f;
          s2[c][b] = half2v{(_Float16)sv, (_Float16)sv};
        }
      }
    };
    auto load_a = [&](int q, uint4* st) {
      // K tail (K not a multiple of KC): the piece is clamped to the row's last
      // one; its weights carry scale 0 there
      const int kk = min(q * KC + grp8, K - 8);
#pragma unroll
      for (int i = 0; i < NST; ++i)
        st[i] = order_for_b<SCHEME>(load8_f16<MODE == 1 ? MOE_F16 : XT>(Ab + aoff[i], kk));
    };
    for (int q = 0; q < nchunks; ++q) {
      Block<SCHEME> wb[2][BPG];
      half2v s2[2][BPG];
      uint4 st[NST];
      load_w(q, wb, s2);
      load_a(q, st);
      __syncthreads();  // previous chunk's MFMAs are done with As
#pragma unroll
      for (int i = 0; i < NST; ++i)
        *reinterpret_cast<uint4*>(As + (tid / PPR + i * (256 / PPR)) * AROW + grp8 * 2) = st[i];
      __syncthreads();
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        half8v b[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) b[c] = block_slice_f16<SCHEME>(wb[c][j / 4], j % 4, s2[c][j / 4]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (mt < mtiles) {
            // A: row mt*16 + r16, chunk elements 32*BPG*g + 8j .. +7
            const half8v a =
                *reinterpret_cast<const half8v*>(As + (mt * 16 + r16) * AROW + (32 * BPG * g + 8 * j) * 2);
#pragma unroll
            for (int c = 0; c < 2; ++c)
              acc[mt][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[c], acc[mt][c], 0, 0, 0);
          }
        }
      }
    }
    // epilogue: lane holds rows m = mt*16 + 4g + i, column col[c] + r16
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mt * 16 + 4 * g + i;
        if (m >= nm) continue;
        const int f = fs[m];
        if (MODE == 0) {
          const int n = col[0] + r16;
          if (n < lim) {
            const float hv = silu(acc[mt][0][i]) * acc[mt][1][i];
            h16[(int64_t)f * I + n] = __builtin_bit_cast(uint16_t, (_Float16)hv);
          }
        } else {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int n = col[c] + r16;
            if (n < lim) ys[(int64_t)f * H + n] = acc[mt][c][i];
          }
        }
      }
    }
  }
}

hipError_t launch_gemm_grouped(const void* x, int xtype, int T, const ExpertsDev& ex, int k, const GroupBufs& g,
                               const float* gate, uint16_t* h16, float* ys, float* y, hipStream_t s) {
  const int maxu = (int)std::min<int64_t>((int64_t)ex.E, (int64_t)T * k);
  const double avg = (double)T * k / ex.E;
  auto run = [&](auto SC, auto XC, auto MTc) {
    constexpr int S_ = decltype(SC)::value, X_ = decltype(XC)::value, MT_ = decltype(MTc)::value;
    dim3 g1((ex.I + 63) / 64, maxu), g2((ex.H + 127) / 128, maxu);
    MOE_LAUNCH(MOE_KERNEL_GEMM_GATE_UP, (k_gemm_grouped<S_, X_, 0, MT_>), g1, dim3(256), 0, s, x, ex, k, g.uniq,
               g.n_uniq, g.counts, g.offsets, g.perm, h16, ys);
    MOE_LAUNCH(MOE_KERNEL_GEMM_DOWN, (k_gemm_grouped<S_, MOE_F16, 1, MT_>), g2, dim3(256), 0, s,
               (const void*)h16, ex, k, g.uniq, g.n_uniq, g.counts, g.offsets, g.perm, h16,
               gate ? ys : y);
  };
  auto with_mt = [&](auto SC, auto XC) {
    if (avg > 24) run(SC, XC, ICg<8>{});
    else if (avg > 6) run(SC, XC, ICg<4>{});
    else run(SC, XC, ICg<1>{});
  };
  auto with_x = [&](auto SC) {
    if (xtype == MOE_F32) with_mt(SC, ICg<MOE_F32>{});
    else if (xtype == MOE_F16) with_mt(SC, ICg<MOE_F16>{});
    else with_mt(SC, ICg<MOE_BF16>{});
  };
  if (ex.scheme == MOE_Q_SYM8) with_x(ICg<MOE_Q_SYM8>{});
  else with_x(ICg<MOE_Q_INT4>{});
  if (gate) return launch_combine(T, ex.H, k, gate, ys, y, s);
  return hipGetLastError();
}

}  // namespace moe
