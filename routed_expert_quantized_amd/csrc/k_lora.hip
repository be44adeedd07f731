// Block-quantized linear with an unmerged LoRA delta.
// "The Other Half of the Memory Wall: Serving 35B MoEs from SSD with Trained
// Routing Prediction" (xyznot.com), section 手法 (method), "非マージアダプターの
// 実行": the layer keeps its quantized base bytes and runs the low-rank delta
// beside them, y = W_q x + (alpha / r) B A x; section よくある質問 (FAQ): merging
// the delta into 4-bit weights and re-quantising loses most of it.
//
// Two launches. The first makes u = A x (r values per token; A is small and
// read once). The second is the quantized matvec (one row per wave for a single
// token, several for a batch; from 16 fp16 tokens a matrix-core tile), with the
// delta folded into the same wave-wide sum:
// lanes 0..r-1 each add scale * B[n][j] * u[j] to their partial before the
// reduction, so the delta costs r floats of B per row and no extra pass over y.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kLoraWaves = 4;

// u[t][j] = A[j] . x_t: one workgroup per adapter row j and group of TU tokens,
// the row in registers, wave w owning the 256-column chunks w, w + 4, ...
template <int XT, int NCH, int TU>
__global__ __launch_bounds__(64 * kLoraWaves) void k_lora_a(const void* __restrict__ x, int T, int K,
                                                           const float* __restrict__ A, int r,
                                                           float* __restrict__ u) {
  __shared__ float red[kLoraWaves][TU];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = blockIdx.x;
  const int t0 = blockIdx.y * TU;
  const int nx = (K + 255) >> 8;
  const float* row = A + (int64_t)j * K;
  float4 wr[NCH];
  int col[NCH];
  bool ok[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = w + kLoraWaves * i;
    const int q = c * 256 + lane * 4;
    ok[i] = c < nx && q < K;
    col[i] = min(q, K - 4);  // in bounds; masked out of the sums when !ok
    wr[i] = *reinterpret_cast<const float4*>(row + col[i]);
  }
#pragma unroll
  for (int v = 0; v < TU; ++v) {
    const int t = min(t0 + v, T - 1);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (ok[i]) {
        const float4 xv = load_x4<XT>(x, (int64_t)t * K + col[i]);
        acc = fmaf(wr[i].x, xv.x, acc);
        acc = fmaf(wr[i].y, xv.y, acc);
        acc = fmaf(wr[i].z, xv.z, acc);
        acc = fmaf(wr[i].w, xv.w, acc);
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) red[w][v] = acc;
  }
  __syncthreads();
  if (w == 0 && lane < TU && t0 + lane < T) {
    float z = 0.0f;
#pragma unroll
    for (int q = 0; q < kLoraWaves; ++q) z += red[q][lane];
    u[(int64_t)(t0 + lane) * r + j] = z;
  }
}

// y[t][n] = sum over blocks b of scale[n][b] * (codes[n][b] . x_t[b])
//           + c * sum_j B[n][j] u[t][j]
// Each wave owns RPW consecutive rows; lane l holds blocks l, l + 64, ... (BPL
// of them) of every row in registers, and each x block it loads serves all RPW
// rows. blockIdx.y takes TG consecutive tokens.
template <int SCHEME, int XT, int BPL, int RPW>
__global__ __launch_bounds__(64 * kLoraWaves) void k_qlinear_lora(
    const void* __restrict__ x, int T, int TG, int N, int K, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const float* __restrict__ u, const float* __restrict__ B, int r, float c,
    float* __restrict__ y) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * kLoraWaves + w) * RPW;
  if (n0 >= N) return;
  const int nb = K >> 5;
  Block<SCHEME> blk[RPW][BPL];
  float sc[RPW][BPL];
  float bj[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    const int n = min(n0 + q, N - 1);  // rows past N repeat the last row and are not stored
    const uint8_t* crow = codes + (int64_t)n * row_bytes<SCHEME>(K);
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const int b = lane + 64 * i;
      if (b < nb) {
        blk[q][i] = load_block<SCHEME>(crow, b);
        sc[q][i] = f16_bits_to_f32(scales[(int64_t)n * nb + b]);
      } else {
        sc[q][i] = 0.0f;
      }
    }
    bj[q] = lane < r ? c * B[(int64_t)n * r + lane] : 0.0f;
  }
  const int t0 = blockIdx.y * TG, t1 = min(t0 + TG, T);
  for (int t = t0; t < t1; ++t) {
    const float ut = lane < r ? u[(int64_t)t * r + lane] : 0.0f;
    float acc[RPW];
#pragma unroll
    for (int q = 0; q < RPW; ++q) acc[q] = bj[q] * ut;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const int b = lane + 64 * i;
      if (b < nb) {
        XReg<SCHEME, XT> xr;
        load_xreg<SCHEME, XT>(xr, x, (int64_t)t * K, b);
#pragma unroll
        for (int q = 0; q < RPW; ++q) acc[q] = fmaf(sc[q][i], xdot<SCHEME, XT>(blk[q][i], xr), acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const float v = wave_sum(acc[q]);
      if (lane == 0 && n0 + q < N) y[(int64_t)t * N + n0 + q] = v;
    }
  }
}

// Batched form for fp16 activations, on the matrix cores. Codes are exact in
// fp16 and the MFMA's K of 32 is one quantisation block, so each block's fp32
// partial is multiplied by its row's scale before it joins the sum: the same
// products and per-block scaling as the matvec, summed in another order. A
// workgroup owns a 16-token x 16-row tile; its four waves split K and add their
// partial tiles in LDS. Operand layout of
// v_mfma_f32_16x16x32_f16: lane l holds A[l%16][8(l/16)+j] and B[8(l/16)+j][l%16]
// for j < 8, and D[4(l/16)+i][l%16] for i < 4; here A = x (token rows), B =
// codes (weight rows as columns), D[token][row].
typedef _Float16 half8_l __attribute__((ext_vector_type(8)));
typedef float float4_l __attribute__((ext_vector_type(4)));

template <int SCHEME>
__device__ __forceinline__ half8_l codes8(const uint8_t* __restrict__ row, int k0) {
  half8_l h;
  if constexpr (SCHEME == MOE_Q_SYM8) {
    const uint2 v = *reinterpret_cast<const uint2*>(row + k0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = (_Float16)(int)(int8_t)(v.x >> (8 * j));
      h[4 + j] = (_Float16)(int)(int8_t)(v.y >> (8 * j));
    }
  } else {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(row + k0 / 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = (_Float16)(((int)(v << (28 - 4 * j))) >> 28);
  }
  return h;
}

template <int SCHEME>
__global__ __launch_bounds__(64 * kLoraWaves) void k_qlinear_lora_mfma(
    const uint16_t* __restrict__ x, int T, int N, int K, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const float* __restrict__ u, const float* __restrict__ B, int r, float c,
    float* __restrict__ y) {
  static_assert(kLoraWaves == 4, "wave w adds the delta of the lane's w-th output row");
  __shared__ float red[kLoraWaves][4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
  const int nb = K >> 5;
  const int n = min(n0 + r16, N - 1);   // rows past N are read in bounds and not stored
  const int ta = min(t0 + r16, T - 1);  // token row of this lane's A operand
  const uint8_t* crow = codes + (int64_t)n * row_bytes<SCHEME>(K);
  const uint16_t* srow = scales + (int64_t)n * nb;
  const uint16_t* xrow = x + (int64_t)ta * K;
  // the delta of token t0 + 4g + w for this lane's row, before the products so
  // its loads overlap them; wave w adds it to output i == w
  const int td = min(t0 + 4 * g + w, T - 1);
  float d = 0.0f;
#pragma unroll 8
  for (int j = 0; j < r; ++j) d = fmaf(B[(int64_t)n * r + j], u[(int64_t)td * r + j], d);
  // wave w takes blocks [b0, b1) of K
  const int per = (nb + kLoraWaves - 1) / kLoraWaves;
  const int b0 = w * per, b1 = min(nb, b0 + per);
  float4_l acc = {0.f, 0.f, 0.f, 0.f};
  for (int b = b0; b < b1; ++b) {
    const int k0 = 32 * b + 8 * g;
    const half8_l a = __builtin_bit_cast(half8_l, *reinterpret_cast<const uint4*>(xrow + k0));
    const half8_l bq = codes8<SCHEME>(crow, k0);
    const float4_l p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq, float4_l{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    const float s = f16_bits_to_f32(srow[b]);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(s, p[i], acc[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[w][i][lane] = i == w ? fmaf(c, d, acc[i]) : acc[i];
  __syncthreads();
  if (w != 0) return;
  const bool store = n0 + r16 < N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = red[0][i][lane];
#pragma unroll
    for (int q = 1; q < kLoraWaves; ++q) v += red[q][i][lane];
    const int t = t0 + 4 * g + i;
    if (store && t < T) y[(int64_t)t * N + n] = v;
  }
}

}  // namespace

hipError_t launch_qlinear_lora(const void* x, int xtype, int T, int N, int K, int scheme, const uint8_t* codes,
                               const uint16_t* scales, const float* A, const float* B, int r, float c, float* u,
                               float* y, hipStream_t s) {
  if (r > 0) {
    const int nch = ((K + 255) / 256 + kLoraWaves - 1) / kLoraWaves;
    auto go = [&](auto NC, auto TUc) {
      constexpr int NN = decltype(NC)::value, U = decltype(TUc)::value;
      const dim3 grid(r, (T + U - 1) / U), block(64 * kLoraWaves);
      switch (xtype) {
        case MOE_F32: MOE_LAUNCH(MOE_KERNEL_LORA, (k_lora_a<MOE_F32, NN, U>), grid, block, 0, s, x, T, K, A, r, u); break;
        case MOE_F16: MOE_LAUNCH(MOE_KERNEL_LORA, (k_lora_a<MOE_F16, NN, U>), grid, block, 0, s, x, T, K, A, r, u); break;
        default:      MOE_LAUNCH(MOE_KERNEL_LORA, (k_lora_a<MOE_BF16, NN, U>), grid, block, 0, s, x, T, K, A, r, u); break;
      }
    };
    auto with_tu = [&](auto NC) {
      if (T == 1) go(NC, std::integral_constant<int, 1>{});
      else go(NC, std::integral_constant<int, 4>{});
    };
    if (nch <= 1) with_tu(std::integral_constant<int, 1>{});
    else if (nch <= 2) with_tu(std::integral_constant<int, 2>{});
    else with_tu(std::integral_constant<int, 4>{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (xtype == MOE_F16 && T >= 16) {
    const dim3 grid((N + 15) / 16, (T + 15) / 16), block(64 * kLoraWaves);
    const uint16_t* xh = static_cast<const uint16_t*>(x);
    if (scheme == MOE_Q_SYM8)
      MOE_LAUNCH(MOE_KERNEL_LORA, k_qlinear_lora_mfma<MOE_Q_SYM8>, grid, block, 0, s, xh, T, N, K, codes, scales, u, B, r, c, y);
    else
      MOE_LAUNCH(MOE_KERNEL_LORA, k_qlinear_lora_mfma<MOE_Q_INT4>, grid, block, 0, s, xh, T, N, K, codes, scales, u, B, r, c, y);
    return hipGetLastError();
  }
  const int bpl = (K / 32 + 63) / 64;
  // one row per wave for a single token (most workgroups); for a batch, 4 rows
  // per wave (2 for K > 2048) share each x block and a workgroup takes 16 tokens
  const int tg = T == 1 ? 1 : 16;
  auto go = [&](auto SC, auto XC, auto BC, auto RC) {
    constexpr int S = decltype(SC)::value, X = decltype(XC)::value, BP = decltype(BC)::value,
                  R = decltype(RC)::value;
    const dim3 grid((N + kLoraWaves * R - 1) / (kLoraWaves * R), (T + tg - 1) / tg), block(64 * kLoraWaves);
    MOE_LAUNCH(MOE_KERNEL_LORA, (k_qlinear_lora<S, X, BP, R>), grid, block, 0, s, x, T, tg, N, K, codes, scales, u,
               B, r, c, y);
  };
  auto with_rows = [&](auto SC, auto XC, auto BC) {
    constexpr int RB = decltype(BC)::value == 1 ? 4 : 2;  // rows per wave within the register budget
    if (T == 1) go(SC, XC, BC, std::integral_constant<int, 1>{});
    else go(SC, XC, BC, std::integral_constant<int, RB>{});
  };
  auto with_b = [&](auto SC, auto XC) {
    if (bpl <= 1) with_rows(SC, XC, std::integral_constant<int, 1>{});
    else with_rows(SC, XC, std::integral_constant<int, 2>{});
  };
  auto with_x = [&](auto SC) {
    switch (xtype) {
      case MOE_F32: with_b(SC, std::integral_constant<int, MOE_F32>{}); break;
      case MOE_F16: with_b(SC, std::integral_constant<int, MOE_F16>{}); break;
      default: with_b(SC, std::integral_constant<int, MOE_BF16>{}); break;
    }
  };
  if (scheme == MOE_Q_SYM8) with_x(std::integral_constant<int, MOE_Q_SYM8>{});
  else with_x(std::integral_constant<int, MOE_Q_INT4>{});
  return hipGetLastError();
}

}  // namespace moe
