// common.hpp — device helpers shared by the gfx950 kernels of the MoE expert layer.
//
// Pages cited (title, then the section):
//   [LR] "QwenのMoEルーターを観測してホットエキスパートを先読みしても速くならなかった" (lilting.ch)
//   [QK] "鳴かぬなら、カスタムカーネル、ほととぎす" (qiita.com, john-rocky)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = WIDTH / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// ---------------------------------------------------------------- number formats
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Order-preserving map of an fp32 value onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float float_from_order_key(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __builtin_bit_cast(float, u);
}

// Load 4 consecutive activations starting at element i (i a multiple of 4), as fp32.
template <int XT>
__device__ __forceinline__ float4 load_x4(const void* x, int64_t i) {
  if constexpr (XT == MOE_F32) {
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + i);
  } else {
    uint2 r = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + i);
    if constexpr (XT == MOE_F16) {
      return make_float4(f16_bits_to_f32((uint16_t)(r.x & 0xFFFF)), f16_bits_to_f32((uint16_t)(r.x >> 16)),
                         f16_bits_to_f32((uint16_t)(r.y & 0xFFFF)), f16_bits_to_f32((uint16_t)(r.y >> 16)));
    } else {
      return make_float4(bf16_bits_to_f32((uint16_t)(r.x & 0xFFFF)), bf16_bits_to_f32((uint16_t)(r.x >> 16)),
                         bf16_bits_to_f32((uint16_t)(r.y & 0xFFFF)), bf16_bits_to_f32((uint16_t)(r.y >> 16)));
    }
  }
}

// Load the 32 activations of quantisation block b (elements 32b .. 32b+31) as fp32.
template <int XT>
__device__ __forceinline__ void load_x_block(const void* x, int64_t row_base, int b, float* xf) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float4 v = load_x4<XT>(x, row_base + 32 * b + 4 * i);
    xf[4 * i + 0] = v.x; xf[4 * i + 1] = v.y; xf[4 * i + 2] = v.z; xf[4 * i + 3] = v.w;
  }
}

// ---------------------------------------------------------------- packed code blocks
// A block is the 32 codes of one row that share a scale [QK §6]. sym8 stores one
// int8 per code (32 bytes a block); int4 stores two codes per byte, the even
// index in the low nibble (16 bytes a block).
template <int SCHEME>
struct Block {
  static constexpr int kBytes = SCHEME == MOE_Q_SYM8 ? 32 : 16;
  static constexpr int kWords = kBytes / 4;
  uint32_t w[kWords];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte loads: expert codes are read once per call.
template <int SCHEME>
__device__ __forceinline__ Block<SCHEME> load_block(const uint8_t* row, int b) {
  Block<SCHEME> blk;
  const u32x4* p = reinterpret_cast<const u32x4*>(row + (int64_t)b * Block<SCHEME>::kBytes);
#pragma unroll
  for (int i = 0; i < Block<SCHEME>::kWords / 4; ++i) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    blk.w[4 * i + 0] = v.x; blk.w[4 * i + 1] = v.y; blk.w[4 * i + 2] = v.z; blk.w[4 * i + 3] = v.w;
  }
  return blk;
}

// Code j (0..31) of a block, sign-extended.
template <int SCHEME>
__device__ __forceinline__ int block_code(const Block<SCHEME>& blk, int j) {
  if constexpr (SCHEME == MOE_Q_SYM8) {
    return (int)(int8_t)(blk.w[j >> 2] >> (8 * (j & 3)));
  } else {
    return ((int)(blk.w[j >> 3] << (28 - 4 * (j & 7)))) >> 28;
  }
}

// sum_j code_j * v_j over the 32 codes of a block, in fp32 (scale not applied).
template <int SCHEME>
__device__ __forceinline__ float block_dot(const Block<SCHEME>& blk, const float* v) {
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) acc = fmaf((float)block_code<SCHEME>(blk, j), v[j], acc);
  return acc;
}

// ---------------------------------------------------------------- routing
// One wave chooses the top k of E logits [LR "ルーターをフックする"]: k rounds of a
// wave-wide argmax over 64-bit keys (order-preserving logit bits, then the
// complement of the expert id, so equal logits go to the lower id). Lane s < k
// returns slot s's expert and gate. Gates are softmax probabilities, computed
// relative to the largest logit; with renorm they are divided by their sum
// over the k chosen, otherwise by the sum over all E.
template <int VPL>
__device__ __forceinline__ void wave_topk(const float* logits, int E, int k, bool renorm,
                                          int& my_idx, float& my_gate) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = lane + kWave * j;
    v[j] = e < E ? logits[e] : 0.0f;
  }
  uint32_t taken = 0;
  my_idx = -1;
  float my_logit = 0.0f, lmax = 0.0f;
  for (int s = 0; s < k; ++s) {
    int bj = -1;
    float bv = 0.0f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = lane + kWave * j;
      if (e < E && !((taken >> j) & 1u) && (bj < 0 || v[j] > bv)) { bj = j; bv = v[j]; }
    }
    uint64_t key = 0;
    if (bj >= 0) {
      const uint32_t e = (uint32_t)(lane + kWave * bj);
      key = ((uint64_t)float_order_key(bv) << 32) | (uint64_t)(0xFFFFFFFFu - e);
    }
    key = wave_max_u64(key);
    const int win = (int)(0xFFFFFFFFu - (uint32_t)key);
    const float wv = float_from_order_key((uint32_t)(key >> 32));
    if ((win & (kWave - 1)) == lane) taken |= 1u << (win / kWave);
    if (s == 0) lmax = wv;
    if (lane == s) { my_idx = win; my_logit = wv; }
  }
  float denom;
  if (renorm) {
    float p = lane < k ? expf(my_logit - lmax) : 0.0f;
    denom = wave_sum(p);
  } else {
    float p = 0.0f;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (lane + kWave * j < E) p += expf(v[j] - lmax);
    denom = wave_sum(p);
  }
  my_gate = lane < k ? expf(my_logit - lmax) / denom : 0.0f;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

}  // namespace moe
