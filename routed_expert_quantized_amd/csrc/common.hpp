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

// ---------------------------------------------------------------- cross-lane
// DPP moves within a 16-lane row (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror,
// row_mirror): after the four steps every lane of a row holds the row's result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return v;
}

__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}

__device__ __forceinline__ int row_min16(int v) {
  v = min(v, dpp_i<kDppXor1>(v));
  v = min(v, dpp_i<kDppXor2>(v));
  v = min(v, dpp_i<kDppHalfMirror>(v));
  v = min(v, dpp_i<kDppMirror>(v));
  return v;
}

// Combine the four 16-lane rows: v_permlane16_swap pairs rows (0,1) and (2,3),
// then v_permlane32_swap pairs the two halves. Element 0 of each result holds
// the lower row/half and element 1 the upper one, in every lane, so the wave
// result ends up in a VGPR of every lane without a round trip through SGPRs.
// The two halves pass through an empty asm statement: without it the compiler
// has been seen to treat the two results of a swap of one value as equal.
__device__ __forceinline__ void swap16(uint32_t v, uint32_t& lo, uint32_t& hi) {
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  lo = r[0];
  hi = r[1];
  asm volatile("" : "+v"(lo), "+v"(hi));
}
__device__ __forceinline__ void swap32(uint32_t v, uint32_t& lo, uint32_t& hi) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  lo = r[0];
  hi = r[1];
  asm volatile("" : "+v"(lo), "+v"(hi));
}

__device__ __forceinline__ float wave_sum(float v) {
  uint32_t a, b;
  v = row_sum16(v);
  swap16(__builtin_bit_cast(uint32_t, v), a, b);
  v = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  swap32(__builtin_bit_cast(uint32_t, v), a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

__device__ __forceinline__ float wave_max(float v) {
  uint32_t a, b;
  v = row_max16(v);
  swap16(__builtin_bit_cast(uint32_t, v), a, b);
  v = fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  swap32(__builtin_bit_cast(uint32_t, v), a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

__device__ __forceinline__ int wave_min_i(int v) {
  uint32_t a, b;
  v = row_min16(v);
  swap16((uint32_t)v, a, b);
  v = min((int)a, (int)b);
  swap32((uint32_t)v, a, b);
  return min((int)a, (int)b);
}

// Sum over aligned groups of 16 lanes; every lane of the group gets it.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(WIDTH == 16, "only 16-lane groups");
  return row_sum16(v);
}

// ---------------------------------------------------------------- number formats
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// fp16 scale at p, or +0 where keep is false (whatever p holds, NaN included).
// The load is issued whatever keep says and the bits are masked: a select
// between the loaded value and 0 is compiled into a branch around the load,
// with a wait for it inside, which serialises a kernel's loads; the empty asm
// hides from the optimiser that the mask is one of two constants.
__device__ __forceinline__ float scale_or_zero(const uint16_t* p, bool keep) {
  uint32_t m = keep ? 0xFFFFu : 0u;
  asm("" : "+v"(m));
  return f16_bits_to_f32((uint16_t)(*p & m));
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

// ---------------------------------------------------------------- fp16 activation blocks
// For fp16 activations the dot runs as v_dot2_f32_f16: codes become exact fp16
// pairs (a code c in [-128, 127] is (1024 + (c + 128)) - 1152 in fp16, built with
// one byte permute and one packed half subtraction), products are exact and
// the sum is fp32.
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }

// 32 fp16 activations of one block as 16 packed pairs. For int4 the pairs are
// reordered to (x[8i+j], x[8i+j+4]) to match the nibble unpacking below.
template <int SCHEME>
struct XBlockH {
  uint32_t p[16];
};

template <int SCHEME>
__device__ __forceinline__ XBlockH<SCHEME> xblock_from_pairs(const uint32_t* nat) {
  XBlockH<SCHEME> xb;
  if constexpr (SCHEME == MOE_Q_SYM8) {
#pragma unroll
    for (int i = 0; i < 16; ++i) xb.p[i] = nat[i];
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g) {  // 8 activations per 32-bit code word
      const uint32_t a = nat[4 * g], b = nat[4 * g + 1], c = nat[4 * g + 2], d = nat[4 * g + 3];
      xb.p[4 * g + 0] = __builtin_amdgcn_perm(c, a, 0x05040100u);  // (x0, x4)
      xb.p[4 * g + 1] = __builtin_amdgcn_perm(c, a, 0x07060302u);  // (x1, x5)
      xb.p[4 * g + 2] = __builtin_amdgcn_perm(d, b, 0x05040100u);  // (x2, x6)
      xb.p[4 * g + 3] = __builtin_amdgcn_perm(d, b, 0x07060302u);  // (x3, x7)
    }
  }
  return xb;
}

template <int SCHEME>
__device__ __forceinline__ XBlockH<SCHEME> load_xblock_h(const uint16_t* x, int64_t row_base, int b) {
  uint32_t nat[16];
  const uint4* p = reinterpret_cast<const uint4*>(x + row_base + 32 * b);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = p[i];
    nat[4 * i] = v.x; nat[4 * i + 1] = v.y; nat[4 * i + 2] = v.z; nat[4 * i + 3] = v.w;
  }
  return xblock_from_pairs<SCHEME>(nat);
}

template <int SCHEME>
__device__ __forceinline__ float block_dot_h(const Block<SCHEME>& blk, const XBlockH<SCHEME>& xb) {
  float acc = 0.0f;
  if constexpr (SCHEME == MOE_Q_SYM8) {
    const half2v bias = as_h2(0xE480E480u);  // -1152
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t u = blk.w[i] ^ 0x80808080u;
      const half2v lo = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) + bias;
      const half2v hi = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) + bias;
      acc = __builtin_amdgcn_fdot2(lo, as_h2(xb.p[2 * i]), acc, false);
      acc = __builtin_amdgcn_fdot2(hi, as_h2(xb.p[2 * i + 1]), acc, false);
    }
  } else {
    const half2v bias = as_h2(0xE408E408u);  // -1032
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = blk.w[i] ^ 0x88888888u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t pr = ((u >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
        acc = __builtin_amdgcn_fdot2(as_h2(pr) + bias, as_h2(xb.p[4 * i + j]), acc, false);
      }
    }
  }
  return acc;
}

// ---------------------------------------------------------------- routing
// One wave chooses the top k of E logits [LR "ルーターをフックする"]: k rounds of a
// wave-wide max over each lane's best remaining logit, equal logits going to the
// lower expert id. Lane s < k returns slot s's expert and gate. Gates are
// softmax probabilities taken relative to the largest logit; with renorm they
// are divided by their sum over the k chosen, otherwise by the sum over all E.
template <int VPL>
__device__ __forceinline__ void wave_topk_scan(const float* logits, int E, int k, bool renorm,
                                               int& my_idx, float& my_gate) {
  const int lane = threadIdx.x & (kWave - 1);
  const float kNone = -__builtin_inff();
  float v[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = lane + kWave * j;
    v[j] = e < E ? logits[e] : kNone;
  }
  uint32_t taken = 0;
  // this lane's best remaining value and its expert id (lowest j on ties = lowest id)
  auto best = [&](float& bv, int& be) {
    bv = kNone;
    be = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = lane + kWave * j;
      if (e < E && !((taken >> j) & 1u) && (be == 0x7FFFFFFF || v[j] > bv)) { bv = v[j]; be = e; }
    }
  };
  float cv;
  int ce;
  best(cv, ce);
  my_idx = -1;
  float my_logit = 0.0f, lmax = 0.0f;
  for (int s = 0; s < k; ++s) {
    const float m = wave_max(cv);
    const uint64_t tie = __ballot(cv == m && ce != 0x7FFFFFFF);
    int win;
    if (__popcll(tie) == 1) {
      win = __builtin_amdgcn_readlane(ce, (int)__builtin_ctzll(tie));
    } else {
      win = wave_min_i((cv == m) ? ce : 0x7FFFFFFF);
    }
    if (s == 0) lmax = m;
    if (lane == s) { my_idx = win; my_logit = m; }
    if (ce == win) {
      taken |= 1u << (win / kWave);
      best(cv, ce);
    }
  }
  float p;
  if (renorm) {
    p = lane < k ? expf(my_logit - lmax) : 0.0f;
  } else {
    p = 0.0f;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (lane + kWave * j < E) p += expf(v[j] - lmax);
  }
  const float denom = wave_sum(p);
  my_gate = lane < k ? expf(my_logit - lmax) / denom : 0.0f;
}

// Integer max over the wave (every lane gets it).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<kDppXor1>((int)v));
  v = max(v, (uint32_t)dpp_i<kDppXor2>((int)v));
  v = max(v, (uint32_t)dpp_i<kDppHalfMirror>((int)v));
  v = max(v, (uint32_t)dpp_i<kDppMirror>((int)v));
  uint32_t a, b;
  swap16(v, a, b);
  v = max(a, b);
  swap32(v, a, b);
  return max(a, b);
}

// Order-preserving key of an fp32 value; -0 and +0 map to the same key, as
// they compare equal. 0 is below every key, so it marks an empty entry.
__device__ __forceinline__ uint32_t logit_key(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f) == 0x80000000u ? 0u : __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Top k of E <= 64 * VPL logits with one wave, each lane first sorting its
// VPL (key, id) pairs (larger logit first, lower id first on equal logits).
// Each round takes the wave-wide largest head; the winning lane pops it.
// Same contract as wave_topk_scan.
// Only the first `rounds` slots are produced (lanes s < rounds); gates are
// computed when with_gates is set, and need rounds == k.
// With ROWS, a slot table slot_of [E] comes along: each lane loads its
// experts' entries beside their logits and carries them through the sort, so
// lane s also gets the entry of the expert of rank s in my_row (-1 when it is
// outside [0, nslots)) without a dependent load after the selection.
template <int VPL, bool ROWS = false>
__device__ __forceinline__ void wave_topk_sorted(const float* logits, int E, int k, bool renorm,
                                                 int& my_idx, float& my_gate, int rounds, bool with_gates,
                                                 const int32_t* slot_of = nullptr, int nslots = 0,
                                                 int* my_row = nullptr) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[VPL];
  uint32_t key[VPL];
  int id[VPL], sl[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = lane + kWave * j;
    // read in bounds whatever e is (a load under a condition becomes a branch)
    v[j] = logits[min(e, E - 1)];
    if constexpr (ROWS) sl[j] = slot_of[min(e, E - 1)];
  }
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = lane + kWave * j;
    key[j] = e < E ? logit_key(v[j]) : 0u;
    id[j] = e;
  }
  // Insertion network, larger key first. A lane's ids grow with j, and an entry
  // only moves past strictly smaller keys, so equal keys keep the lower id
  // first without comparing ids.
#pragma unroll
  for (int a = 1; a < VPL; ++a)
#pragma unroll
    for (int b = a; b > 0; --b) {
      const bool sw = key[b] > key[b - 1];
      const uint32_t k0 = key[b - 1], k1 = key[b];
      const int i0 = id[b - 1], i1 = id[b];
      key[b - 1] = sw ? k1 : k0; key[b] = sw ? k0 : k1;
      id[b - 1] = sw ? i1 : i0; id[b] = sw ? i0 : i1;
      if constexpr (ROWS) {
        const int r0 = sl[b - 1], r1 = sl[b];
        sl[b - 1] = sw ? r1 : r0; sl[b] = sw ? r0 : r1;
      }
    }
  my_idx = -1;
  my_gate = 0.0f;
  uint32_t my_key = 0, kmax = 0;
  // The sorted entries stay in place: `head` counts the lane's entries already
  // taken, and each round reads the new head with one compare and two selects
  // per entry. (Shifting the arrays on every pop is turned by the compiler into
  // selects over every position, several times the work.) An exhausted lane
  // offers key 0, below every logit.
  int head = 0;
  uint32_t hk = key[0];
  int hid = id[0], hsl = ROWS ? sl[0] : 0, row = -1;
  for (int s = 0; s < rounds; ++s) {
    const uint32_t m = wave_max_u32(hk);
    const uint64_t tie = __ballot(hk == m);
    int win;
    if constexpr (ROWS) {
      // the winning lane: the only one holding the maximum, else the one
      // among them with the lowest id
      int wl = (int)__builtin_ctzll(tie);
      if (__popcll(tie) != 1) {
        const int lo = wave_min_i(hk == m ? hid : 0x7FFFFFFF);
        wl = (int)__builtin_ctzll(__ballot(hk == m && hid == lo));
      }
      win = __builtin_amdgcn_readlane(hid, wl);
      const int r = __builtin_amdgcn_readlane(hsl, wl);
      if (lane == s) row = r;
    } else {
      if (__popcll(tie) == 1) win = __builtin_amdgcn_readlane(hid, (int)__builtin_ctzll(tie));
      else win = wave_min_i(hk == m ? hid : 0x7FFFFFFF);
    }
    if (s == 0) kmax = m;
    if (lane == s) { my_idx = win; my_key = m; }
    head += hid == win ? 1 : 0;
    hk = 0u;
    hid = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      hk = head == j ? key[j] : hk;
      hid = head == j ? id[j] : hid;
      if constexpr (ROWS) hsl = head == j ? sl[j] : hsl;
    }
  }
  if constexpr (ROWS) *my_row = row >= 0 && row < nslots ? row : -1;
  if (!with_gates) return;
  const float lmax = key_logit(kmax);
  const float my_logit = key_logit(my_key);
  float p;
  if (renorm) {
    p = lane < k ? expf(my_logit - lmax) : 0.0f;
  } else {
    p = 0.0f;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (lane + kWave * j < E) p += expf(v[j] - lmax);
  }
  const float denom = wave_sum(p);
  my_gate = lane < k ? expf(my_logit - lmax) / denom : 0.0f;
}

// Top k with gates (lanes s < k hold slot s). With rounds < k only the first
// `rounds` slots are produced and no gates (the scan form produces all k);
// gates = false skips them also at rounds == k.
// With ROWS, lane s also gets the slot-table entry of its expert (as in
// wave_topk_sorted; the scan form looks it up after the selection).
template <int VPL, bool ROWS = false>
__device__ __forceinline__ void wave_topk(const float* logits, int E, int k, bool renorm, int& my_idx,
                                          float& my_gate, int rounds = -1, const int32_t* slot_of = nullptr,
                                          int nslots = 0, int* my_row = nullptr, bool gates = true) {
  if (rounds < 0) rounds = k;
  if constexpr (VPL <= 8) {
    wave_topk_sorted<VPL, ROWS>(logits, E, k, renorm, my_idx, my_gate, rounds, gates && rounds == k, slot_of,
                                nslots, my_row);
  } else {
    wave_topk_scan<VPL>(logits, E, k, renorm, my_idx, my_gate);
    if constexpr (ROWS) {
      const int lane = threadIdx.x & (kWave - 1);
      const int r = lane < k ? slot_of[my_idx] : -1;
      *my_row = r >= 0 && r < nslots ? r : -1;
    }
  }
}

template <int SCHEME>
__host__ __device__ constexpr int64_t row_bytes(int K) {
  return SCHEME == MOE_Q_SYM8 ? (int64_t)K : (int64_t)K / 2;
}

// Activations of one quantisation block, held in registers across rows: fp16
// pairs for the v_dot2 path, fp32 otherwise.
template <int SCHEME, int XT>
struct XReg {
  XBlockH<SCHEME> h;
  float f[32];
};

template <int SCHEME, int XT>
__device__ __forceinline__ void load_xreg(XReg<SCHEME, XT>& r, const void* x, int64_t row_base, int b) {
  if constexpr (XT == MOE_F16) r.h = load_xblock_h<SCHEME>(reinterpret_cast<const uint16_t*>(x), row_base, b);
  else load_x_block<XT>(x, row_base, b, r.f);
}

template <int SCHEME, int XT>
__device__ __forceinline__ void zero_xreg(XReg<SCHEME, XT>& r) {
  if constexpr (XT == MOE_F16) {
#pragma unroll
    for (int i = 0; i < 16; ++i) r.h.p[i] = 0u;
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) r.f[i] = 0.0f;
  }
}

template <int SCHEME, int XT>
__device__ __forceinline__ float xdot(const Block<SCHEME>& c, const XReg<SCHEME, XT>& r) {
  if constexpr (XT == MOE_F16) return block_dot_h<SCHEME>(c, r.h);
  else return block_dot<SCHEME>(c, r.f);
}

// silu(z) = z * sigmoid(z), with the hardware exponential and reciprocal
// (about 1 ulp each); exp overflow for very negative z gives 0.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

}  // namespace moe
