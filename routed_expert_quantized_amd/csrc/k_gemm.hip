// k_gemm.hip — grouped MFMA GEMM for batched tokens (prefill and batched decode).
//
// After the token-by-expert grouping each routed expert e has n_e assignments.
// GEMM1: U_e[n_e][2I] = X_e[n_e][H] . W_gu[e]^T, then h = silu(gate) * up
//        (gate columns n and up columns I + n in the same workgroup).
// GEMM2: Y_e[n_e][H] = h_e[n_e][I] . W_d[e]^T, stored per assignment (ys,
//        ahead of the combine) in fp32, or, where fp32 rows would exceed the
//        256 MB last-level cache, in fp16 with a power of two per row and 32
//        columns (as h below); in per-slot mode into y itself, in fp32.
// Each expert's weights are read once per pass over its assignments
// ("鳴かぬなら、カスタムカーネル、ほととぎす", section 4: only routed experts are read;
// section 7: each slot's down projection takes that slot's own activation).
//
// Arithmetic. Weights enter the matrix cores as their raw codes, which are
// exact in fp16 and bf16, and the K of one v_mfma_f32_16x16x32 is one
// quantisation block (section 6: one scale per 32 K elements). Each block's
// fp32 partial product is multiplied by its row's scale and added to an fp32
// accumulator: the dequantised weight code * scale is never rounded. The
// activations are the MFMA's other operand in their own 16-bit type, fp16 or
// bf16, unconverted. fp32 activations do not take this path.
// h is the down GEMM's activation, stored in fp16 (one rounding) with a power
// of two per tile: the gate/up epilogue takes the largest |h| of its tile (the
// pass's rows x 64 columns) and stores h * 2^-sigma with that maximum in
// [2^14, 2^15), and records sigma; the down GEMM multiplies each block's scale
// by 2^sigma of the block's 64 columns. The powers of two are exact, so h has
// fp16's precision whatever its magnitude.
//
// Operand layout of v_mfma_f32_16x16x32_{f16,bf16} (checked on gfx950): lane l
// holds A[l%16][8(l/16)+j] and B[8(l/16)+j][l%16] for j < 8, and
// D[4(l/16)+i][l%16] for i < 4. Here A = activation rows (assignments), B =
// codes (weight rows as columns), and lane group g = l/16 supplies elements
// 8g .. 8g+7 of the block to both operands. int4 codes unpack as the pairs
// (c_p, c_{p+4}) of a 32-bit word, so for int4 the activations are permuted the
// same way before they reach the MFMA.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "kernels.hpp"
#include "stamps.hpp"

namespace moe {

#ifdef MOE_STAMPS
// Timestamp build only. Per kernel mode (0 gate/up, 1 down) of k_gemm_dma, the
// waves' shader-clock cycles summed by phase: 0 DMA wait, 1 barrier, 2 issue
// + compute, 3 whole wave, 4 number of waves, 5 pass set-up, 6 prologue
// issue, 7 trailing wait, 8 epilogue, 9 tiles (from a tile's start to the end
// of its last pass), 10 tile set-up.
__device__ unsigned long long g_stamps_gemm[2][16];
#endif

typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int V>
using ICg = std::integral_constant<int, V>;

// The MFMA of one 16x16 tile and one quantisation block, in the activation type.
template <int AT>
struct BlockMfma;
template <>
struct BlockMfma<MOE_F16> {
  typedef half8v v8;
  static __device__ __forceinline__ float4v run(v8 a, v8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, float4v{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
};
template <>
struct BlockMfma<MOE_BF16> {
  typedef bf16x8v v8;
  static __device__ __forceinline__ float4v run(v8 a, v8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, float4v{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
};

// Code words a lane group holds of one block: sym8 codes 8g .. 8g+7 are two
// words (8 bytes); int4 codes 8g .. 8g+7 are word g of the block (4 bytes).
template <int SCHEME>
using CodeWords = std::conditional_t<SCHEME == MOE_Q_SYM8, u32x2, uint32_t>;

// (a & b) | c in one instruction: v_bitop3_b32 with truth table 0xEA (the
// table's bit i is the result for a, b, c = bits 2, 1, 0 of i). Written out
// because VOP3 takes no literal constants: the compiler splits the pair into
// an and and an or around a constant it cannot place.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0xea" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// The lane group's 8 codes of one block as exact AT values: sym8 in natural
// order; int4 as (c0, c4), (c1, c5), (c2, c6), (c3, c7).
template <int SCHEME, int AT>
__device__ __forceinline__ typename BlockMfma<AT>::v8 codes8(CodeWords<SCHEME> w) {
  typename BlockMfma<AT>::v8 r;
  if constexpr (AT == MOE_F16) {
    if constexpr (SCHEME == MOE_Q_SYM8) {
      // code c: the fp16 number 1024 + (c + 128), made by one byte permute into
      // 0x64xx, minus 1152
      const half2v bias = as_h2(0xE480E480u);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t u = w[t] ^ 0x80808080u;
        const half2v lo = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) + bias;
        const half2v hi = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) + bias;
        r[4 * t + 0] = lo[0]; r[4 * t + 1] = lo[1]; r[4 * t + 2] = hi[0]; r[4 * t + 3] = hi[1];
      }
    } else {
      // n = c + 8 in [0, 15]. A nibble in bits 0-3 of a halfword ORed into
      // 0x6400 is the fp16 number 1024 + n: minus 1032. A nibble in bits 4-7
      // is 1024 + 16 n: times 1/16, minus 72 (one packed FMA, exact: every
      // value is a small integer). One shift by 8 serves the other two pairs.
      const half2v lo_bias = as_h2(0xE408E408u);  // -1032
      const half2v hi_mul = as_h2(0x2C002C00u);   // 1/16
      const half2v hi_bias = as_h2(0xD480D480u);  // -72
      const uint32_t u = w ^ 0x88888888u, u8 = u >> 8;
      half2v v[4];
      v[0] = as_h2(and_or(u, 0x000F000Fu, 0x64006400u)) + lo_bias;
      v[1] = __builtin_elementwise_fma(as_h2(and_or(u, 0x00F000F0u, 0x64006400u)), hi_mul, hi_bias);
      v[2] = as_h2(and_or(u8, 0x000F000Fu, 0x64006400u)) + lo_bias;
      v[3] = __builtin_elementwise_fma(as_h2(and_or(u8, 0x00F000F0u, 0x64006400u)), hi_mul, hi_bias);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        r[2 * p] = v[p][0];
        r[2 * p + 1] = v[p][1];
      }
    }
  } else {
    // bf16 holds every integer of magnitude <= 256 exactly
    if constexpr (SCHEME == MOE_Q_SYM8) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) r[4 * t + j] = (__bf16)(float)(int)(int8_t)(w[t] >> (8 * j));
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        r[2 * p] = (__bf16)(float)(((int)(w << (28 - 4 * p))) >> 28);
        r[2 * p + 1] = (__bf16)(float)(((int)(w << (12 - 4 * p))) >> 28);
      }
    }
  }
  return r;
}

// 8 activations (natural order, 16-bit elements) in the order B uses.
template <int SCHEME>
__device__ __forceinline__ u32x4 order_for_b(u32x4 h) {
  if constexpr (SCHEME == MOE_Q_SYM8) {
    return h;
  } else {
    // natural pairs (x0,x1)(x2,x3)(x4,x5)(x6,x7) -> (x0,x4)(x1,x5)(x2,x6)(x3,x7)
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(h[2], h[0], 0x05040100u);
    r[1] = __builtin_amdgcn_perm(h[2], h[0], 0x07060302u);
    r[2] = __builtin_amdgcn_perm(h[3], h[1], 0x05040100u);
    r[3] = __builtin_amdgcn_perm(h[3], h[1], 0x07060302u);
    return r;
  }
}

template <int SCHEME, int AT>
__device__ __forceinline__ typename BlockMfma<AT>::v8 a_operand(u32x4 raw) {
  return __builtin_bit_cast(typename BlockMfma<AT>::v8, order_for_b<SCHEME>(raw));
}

// fp32 value to the 16-bit activation type (round to nearest even), as bits.
template <int AT>
__device__ __forceinline__ uint16_t to_act16(float v) {
  if constexpr (AT == MOE_F16) return __builtin_bit_cast(uint16_t, (_Float16)v);
  else return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Exponent sigma for a tile whose largest |h| is amax: amax * 2^-sigma lies in
// [2^14, 2^15), inside fp16's normal range; 0 for an all-zero (or non-finite) tile.
__device__ __forceinline__ int tile_sigma(float amax) {
  const uint32_t b = __builtin_bit_cast(uint32_t, amax);
  const int e = (int)((b >> 23) & 0xFFu);
  if (e == 0xFF || b == 0u) return 0;
  if (e == 0) return -126 - 14 + (31 - __builtin_clz(b)) - 23;  // subnormal: its leading bit
  return e - 127 - 14;
}

// Tile maximum of |v| over the lanes' valid entries, across the workgroup's
// four waves (every thread gets it); red holds 4 floats of LDS.
__device__ __forceinline__ float workgroup_absmax(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Instruction groups for the scheduler: the next `n` instructions of a kind
// (in the order the calls are made within one scheduling region).
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008;
template <int KIND, int N>
__device__ __forceinline__ void sched_group() {
  __builtin_amdgcn_sched_group_barrier(KIND, N, 0);
}

// acc += s * p for the four outputs a lane holds of one tile.
__device__ __forceinline__ void scaled_add(float4v& acc, float s, float4v p) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = fmaf(s, p[i], acc[i]);
}

// The same for the first NR of them (rows 4g + i, i < NR, of lane group g):
// the others are rows past a one-tile pass's last assignment, never stored.
// p is an MFMA result: with NR < 4 some of its registers are otherwise unused,
// and the compiler may hand them to an inline-asm output (whose hazards it
// does not check) while the MFMA is still writing them. The empty asm keeps
// all four in use until after the first FMA, which waits for the MFMA.
template <int NR>
__device__ __forceinline__ void scaled_add_n(float4v& acc, float s, float4v p) {
#pragma unroll
  for (int i = 0; i < NR; ++i) acc[i] = fmaf(s, p[i], acc[i]);
  if constexpr (NR < 4) asm volatile("" ::"v"(p), "v"(acc[0]));
}

// ---------------------------------------------------------------------------
// Register-staged kernel, for rows with an odd number of 32-element blocks
// (the DMA kernel below moves scales as 4-byte pairs).
// Grid: (column blocks per expert, max unique experts); 256 threads, 4 waves.
// MODE 0 (gate/up): wave w owns gate rows n0+16w.. and up rows I+n0+16w.., a
//   workgroup owns 64 gate/up pairs; output h16[f][n] = fp16(h * 2^-sigma) and
//   sig[P][cb] = sigma, P the pass's first position in the grouped list.
// MODE 1 (down, AT = fp16): wave w owns rows n0+32w .. n0+32w+31 of W_d[e]; a
//   workgroup owns 128 rows; output ys[f][n] (fp32).
// The expert's assignments are taken 16*MT at a time (one pass each), K in
// chunks of four blocks (128 elements).
constexpr int kRegChunk = 128;
constexpr int kMaxSlices = 4096 / 64;  // 64-column slices of h, at most

template <int SCHEME, int AT, int MODE, int MT>
__global__ __launch_bounds__(256) void k_gemm_grouped(const uint16_t* __restrict__ act, ExpertsDev ex, int k,
                                                      const int32_t* __restrict__ uniq,
                                                      const int32_t* __restrict__ n_uniq,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ perm, uint16_t* __restrict__ h16,
                                                      int32_t* __restrict__ sig, float* __restrict__ ys) {
  constexpr int AROW = kRegChunk * 2 + 16;  // bytes per LDS activation row (16-bit + pad)
  __shared__ __attribute__((aligned(16))) uint8_t As[16 * MT * AROW];
  __shared__ int fs[16 * MT];
  __shared__ int sg[kMaxSlices];
  __shared__ float red[4];
  const int u = blockIdx.y;
  if (u >= *n_uniq) return;
  const int tid = (int)threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, r16 = lane & 15;
  const int e = uniq[u], cnt = counts[e], beg = offsets[e];
  const int ew = expert_index(ex, e);       // -1: no slot, contributes nothing
  const bool resident = ew >= 0;  // a slot-less expert: zero scales, whatever slot 0 holds
  const int H = ex.H, I = ex.I;
  const int K = MODE == 0 ? H : I;          // reduction length
  const int NB = K / 32;                    // quantisation blocks per weight row
  const int NROW = MODE == 0 ? 2 * I : H;   // weight rows of this expert
  const int lim = MODE == 0 ? I : H;        // valid output columns
  const uint8_t* W = MODE == 0 ? ex.wgu : ex.wd;
  const uint16_t* S = MODE == 0 ? ex.sgu : ex.sd;
  const int64_t rb = row_bytes<SCHEME>(K);
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
  for (int c = 0; c < 2; ++c) wrow[c] = (int64_t)max(ew, 0) * NROW + min(col[c] + r16, NROW - 1);
  const int nchunks = (K + kRegChunk - 1) / kRegChunk;
  const int nsl = (I + 63) / 64;  // h slices per assignment row
  using M = BlockMfma<AT>;

  for (int m0 = 0; m0 < cnt; m0 += 16 * MT) {
    const int nm = min(16 * MT, cnt - m0);
    __syncthreads();
    if (tid < 16 * MT) fs[tid] = tid < nm ? perm[beg + m0 + tid] : -1;
    if (MODE == 1 && tid < nsl) sg[tid] = sig[(int64_t)(beg + m0) * nsl + tid];
    __syncthreads();
    float4v acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[mt][c] = float4v{0.f, 0.f, 0.f, 0.f};
    constexpr int PPR = kRegChunk / 8;        // 16-byte activation pieces per row per chunk
    constexpr int NST = 16 * MT * PPR / 256;  // pieces per thread per chunk
    static_assert((16 * MT * PPR) % 256 == 0, "activation tile must split evenly over 256 threads");
    const int mtiles = (nm + 15) / 16;
    const int grp8 = (tid % PPR) * 8;
    int64_t aoff[NST];
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int row = tid / PPR + i * (256 / PPR);
      const int f = fs[row] >= 0 ? fs[row] : fs[0];
      aoff[i] = (int64_t)(MODE == 0 ? f / k : f) * K;
    }
    for (int q = 0; q < nchunks; ++q) {
      // this lane group's codes and the scales of its two rows, four blocks
      CodeWords<SCHEME> cw[2][4];
      float sc[2][4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int blk = 4 * q + b;
        const int bc = min(blk, NB - 1);  // blocks past the row end: read in bounds, scale 0
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint8_t* row = W + wrow[c] * rb;
          if constexpr (SCHEME == MOE_Q_SYM8) cw[c][b] = *reinterpret_cast<const u32x2*>(row + 32 * bc + 8 * g);
          else cw[c][b] = *reinterpret_cast<const uint32_t*>(row + 16 * bc + 4 * g);
          sc[c][b] = scale_or_zero(S + wrow[c] * NB + bc, blk < NB && resident);
          // down: h of this block's 64-column slice was stored times 2^-sigma
          if (MODE == 1) sc[c][b] = ldexpf(sc[c][b], sg[blk >> 1]);
        }
      }
      u32x4 st[NST];
      const int kk = min(q * kRegChunk + grp8, K - 8);  // K tail: pieces clamped in the row, weights scaled by 0
#pragma unroll
      for (int i = 0; i < NST; ++i) st[i] = *reinterpret_cast<const u32x4*>(act + aoff[i] + kk);
      __syncthreads();  // the previous chunk's MFMAs are done with As
#pragma unroll
      for (int i = 0; i < NST; ++i)
        *reinterpret_cast<u32x4*>(As + (tid / PPR + i * (256 / PPR)) * AROW + grp8 * 2) = st[i];
      __syncthreads();
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        typename M::v8 bf[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) bf[c] = codes8<SCHEME, AT>(cw[c][b]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (mt < mtiles) {
            const u32x4 raw = *reinterpret_cast<const u32x4*>(As + (mt * 16 + r16) * AROW + (32 * b + 8 * g) * 2);
            const typename M::v8 a = a_operand<SCHEME, AT>(raw);
#pragma unroll
            for (int c = 0; c < 2; ++c) scaled_add(acc[mt][c], sc[c][b], M::run(a, bf[c]));
          }
        }
      }
    }
    // epilogue: lane holds rows m = mt*16 + 4g + i, column col[c] + r16
    if constexpr (MODE == 0) {
      const int n = col[0] + r16;
      float hv[MT][4], amax = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hv[mt][i] = silu(acc[mt][0][i]) * acc[mt][1][i];
          if (mt * 16 + 4 * g + i < nm && n < lim) amax = fmaxf(amax, fabsf(hv[mt][i]));
        }
      const int sigma = tile_sigma(workgroup_absmax(amax, red));
      if (tid == 0) sig[(int64_t)(beg + m0) * nsl + blockIdx.x] = sigma;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mt * 16 + 4 * g + i;
          if (m < nm && n < lim) h16[(int64_t)fs[m] * I + n] = to_act16<MOE_F16>(ldexpf(hv[mt][i], -sigma));
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mt * 16 + 4 * g + i;
          if (m >= nm) continue;
          const int f = fs[m];
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

// ---------------------------------------------------------------------------
// Software-pipelined variant: every operand of a K chunk reaches LDS through
// direct-to-LDS loads (global_load_lds), so up to NS-1 chunks are in flight
// while the MFMAs of the current one run, at no register cost. A stage holds,
// for LB bytes of each of the workgroup's 128 weight rows: the codes, their
// fp16 block scales, and the 16*MT x KC activation tile. Scales move as 4-byte
// pairs, so a row must hold an even number of 32-element blocks (K a multiple
// of 64).
//
// Bank layout: a 16-byte LDS slot of code row r holds piece slot ^ swz_b(r); of
// activation row r, piece slot ^ swz_a(r). The DMA lane that fills a slot
// fetches the matching piece, and the fragment reads of 16 lanes then hit 16
// distinct 16-byte bank groups.

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediates, gfx9 encoding (vmcnt in bits [3:0] and [15:14], expcnt
// in [6:4], lgkmcnt in [11:8]); each leaves the other counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the fence of __syncthreads(), which would also wait
// for every LDS-DMA load in flight. The memory clobbers keep LDS accesses on
// their side of it; callers wait for their own loads first.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void dma16(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 4, 0, 0);
}

// LDS reads of DMA-filled stages go through inline asm: the compiler cannot
// see that they do not alias the loads still filling other stages and would
// otherwise wait for every load in flight. Their results are only valid after
// lds_wait(), which names the destination registers so that no use of them is
// scheduled before it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p);
}
__device__ __forceinline__ void lds_read(uint32_t addr, u32x4& v) { asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr)); }
__device__ __forceinline__ void lds_read(uint32_t addr, u32x2& v) { asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(addr)); }
__device__ __forceinline__ void lds_read(uint32_t addr, uint32_t& v) { asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr)); }

template <typename T, int N>
__device__ __forceinline__ void lds_wait(T (&a)[N]) {
  static_assert(N >= 1 && N <= 8, "register count");
  if constexpr (N == 1) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]));
  else if constexpr (N == 2) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]));
  else if constexpr (N == 3) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]));
  else if constexpr (N == 4) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
  else if constexpr (N == 5)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]));
  else if constexpr (N == 6)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]));
  else if constexpr (N == 7)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7]));
}

template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(ICg<Is>{}), ...);
}
// f(ICg<0>{}), ..., f(ICg<N-1>{}), each with a compile-time index
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Stage geometry. LB bytes of each of the 128 weight rows per stage (64 or
// 128: half or whole cache lines).
template <int SCHEME, int MT, int LB>
struct DmaTile {
  static constexpr int BB = SCHEME == MOE_Q_INT4 ? 16 : 32;  // bytes per 32-element block
  static constexpr int BPS = LB / BB;                        // blocks per row per stage
  static constexpr int KC = 32 * BPS;                        // K per stage
  static constexpr int SB = LB / 16;                         // 16-byte code slots per row
  static constexpr int ARB = KC * 2;                         // activation bytes per row per stage
  static constexpr int SPR = ARB / 16;                       // 16-byte activation slots per row
  static constexpr int RPI = 1024 / ARB;                     // activation rows per DMA instruction
  static constexpr int B_BYTES = 128 * LB;
  // scales and activations are rounded up to whole DMA rounds (1 KiB of 4-byte
  // loads, 4 KiB of 16-byte loads across the four waves); the padding is filled
  // with duplicate loads and never read
  static constexpr int S_BYTES = 128 * BPS * 2 < 1024 ? 1024 : 128 * BPS * 2;
  static constexpr int A_BYTES = (16 * MT * ARB + 4095) / 4096 * 4096;
  static constexpr int STAGE = B_BYTES + S_BYTES + A_BYTES;
  static constexpr int NBI = B_BYTES / 4096;  // DMA instructions per wave per stage
  static constexpr int NSI = S_BYTES / 1024;
  static constexpr int NAI = A_BYTES / 4096;
  static constexpr int NI = NBI + NSI + NAI;
  static_assert(B_BYTES % 4096 == 0 && S_BYTES % 1024 == 0, "whole DMA rounds");
  static_assert(BPS == 2 || BPS == 4 || BPS == 8, "scales of a row per stage are read as one 4, 8 or 16-byte word");
  // a row's BPS scales in one LDS read
  using ScaleWord = std::conditional_t<BPS == 2, uint32_t, std::conditional_t<BPS == 4, u32x2, u32x4>>;
  // the stage's KC/64 tile exponents of h (down GEMM) in one LDS read
  static_assert(KC == 64 || KC == 128 || KC == 256, "whole 64-column slices per stage");
  using SigWord = std::conditional_t<KC == 64, uint32_t, std::conditional_t<KC == 128, u32x2, u32x4>>;
  // slot swizzles: 16 lanes reading one logical slot of 16 consecutive rows hit
  // 16 distinct 16-byte bank groups
  static __device__ __forceinline__ int swz_b(int row) { return LB == 128 ? (row >> 1) & 7 : (row >> 2) & 3; }
  static __device__ __forceinline__ int swz_a(int row) { return SPR == 8 ? (row >> 1) & 7 : row & 15; }
  // LDS byte offset, within a code row, of lane group g's codes of block b
  static __device__ __forceinline__ int code_off(int row, int b, int g) {
    if constexpr (SCHEME == MOE_Q_SYM8) return (((2 * b + (g >> 1)) ^ swz_b(row)) << 4) + 8 * (g & 1);
    else return ((b ^ swz_b(row)) << 4) + 4 * g;
  }
};

template <typename W>
__device__ __forceinline__ int word_at(const W& w, int j) {
  if constexpr (std::is_same_v<W, uint32_t>) return (int)w;
  else return (int)w[j];
}

template <typename W>
__device__ __forceinline__ uint32_t scale_bits(const W& w, int b) {
  uint32_t word;
  if constexpr (std::is_same_v<W, uint32_t>) word = w;
  else word = w[b >> 1];
  return (b & 1) ? word >> 16 : word & 0xFFFFu;
}

// OHALF (down only): the per-slot rows go out as fp16 with a power of two per
// row and 32 columns (o16 and osig) instead of fp32 (ys).
template <int SCHEME, int AT, int MODE, int MT, int NS, int LB, bool OHALF = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MT >= 6 ? 2 : (MT == 1 ? (SCHEME == MOE_Q_SYM8 ? 3 : 2) : 1), 8)))
void k_gemm_dma(const uint16_t* __restrict__ act, ExpertsDev ex, int k, const int32_t* __restrict__ uniq,
                const int32_t* __restrict__ n_uniq, const int32_t* __restrict__ counts,
                const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm, uint16_t* __restrict__ h16,
                int32_t* __restrict__ sig, float* __restrict__ ys, uint16_t* __restrict__ o16,
                int32_t* __restrict__ osig, int ncb) {
  using D = DmaTile<SCHEME, MT, LB>;
  using M = BlockMfma<AT>;
  static_assert((NS - 2) * D::NI < 64, "in-flight loads exceed vmcnt");
  // One LDS array per stage, always addressed with a compile-time stage index.
  __shared__ __attribute__((aligned(16))) uint8_t st0[D::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[D::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[NS > 2 ? D::STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st3[NS > 3 ? D::STAGE : 16];
  auto stage = [&](auto R) -> uint8_t* {
    constexpr int r = decltype(R)::value;
    if constexpr (r == 0) return st0;
    else if constexpr (r == 1) return st1;
    else if constexpr (r == 2) return st2;
    else return st3;
  };
  static_assert(NS >= 2 && NS <= 4, "stage count");
  __shared__ int fs[16 * MT];
  __shared__ __attribute__((aligned(16))) int sg[kMaxSlices];
  __shared__ float red[4];
  // Persistent: the grid holds as many workgroups as fit on the chip at once
  // (a multiple of 8), each taking tiles blockIdx.x, +gridDim.x, ... until the
  // routed experts' tiles run out, so no partly filled last round of
  // workgroups is left. Tile order is XCD-aware: ids go round-robin over the 8
  // XCDs, and tile (expert u, column block cb) has id (u/8)*8*ncb + cb*8 + u%8,
  // so all column blocks of an expert (which read the same activation rows)
  // run on one XCD, with the experts alternating over the XCDs.
  MOE_STAMPS_ONLY(unsigned long long st_ph[11] = {}; const unsigned long long st_t0 = stamp_clock();
                  unsigned long long st_tile = st_t0, st_x = st_t0;)
  const int nu = *n_uniq;
  const int ntiles = ncb * ((nu + 7) / 8 * 8);
  const int tid = (int)threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int rest = tile >> 3;
    const int cb = rest % ncb;
    const int u = (rest / ncb) * 8 + (tile & 7);
    if (u >= nu) continue;
    MOE_STAMPS_ONLY(st_tile = stamp_clock();)
    const int e = uniq[u], cnt = counts[e], beg = offsets[e];
    const int ew = expert_index(ex, e);  // -1: no slot, contributes nothing (index 0, zero scales)
    const bool resident = ew >= 0;  // a slot-less expert: zero scales, whatever slot 0 holds
    const int H = ex.H, I = ex.I;
    const int K = MODE == 0 ? H : I;
    const int NB = K / 32;
    const int NROW = MODE == 0 ? 2 * I : H;
    const int lim = MODE == 0 ? I : H;
    const int rb = (int)row_bytes<SCHEME>(K);
    const uint8_t* Wexp = (MODE == 0 ? ex.wgu : ex.wd) + (int64_t)max(ew, 0) * NROW * rb;
    const uint16_t* Sexp = (MODE == 0 ? ex.sgu : ex.sd) + (int64_t)max(ew, 0) * NROW * NB;
    const int n0 = MODE == 0 ? cb * 64 : cb * 128;
    // workgroup-local weight row lr (0..127) -> row of the expert (clamped in range)
    auto grow = [&](int lr) {
      const int r = MODE == 0 ? (lr < 64 ? n0 + lr : I + n0 + lr - 64) : n0 + lr;
      return min(r, NROW - 1);
    };
    // this lane's rows in the two 16-column tiles of its wave
    int lrow[2];
    lrow[0] = MODE == 0 ? wave * 16 + r16 : wave * 32 + r16;
    lrow[1] = MODE == 0 ? 64 + wave * 16 + r16 : wave * 32 + 16 + r16;

    // DMA sources that stay fixed for the whole tile: code rows and scale rows
    int ro[D::NBI], bcol[D::NBI];
#pragma unroll
    for (int i = 0; i < D::NBI; ++i) {
      const int row = (i * 4 + wave) * (1024 / LB) + lane / D::SB;
      ro[i] = grow(row) * rb;
      bcol[i] = 16 * ((lane % D::SB) ^ D::swz_b(row));
    }
    constexpr int DPR = D::BPS / 2;  // scale dwords per row per stage
    int so[D::NSI], sp[D::NSI];
#pragma unroll
    for (int i = 0; i < D::NSI; ++i) {
      const int d = (i * 4 + wave) * 64 + lane;
      so[i] = grow(min(d / DPR, 127)) * NB;
      sp[i] = 2 * (d % DPR);
    }
    const int nchunks = (NB + D::BPS - 1) / D::BPS;
    const int nsl = I / 64;  // h slices per assignment row (I is a multiple of 64 here)

    for (int m0 = 0; m0 < cnt; m0 += 16 * MT) {
      const int nm = min(16 * MT, cnt - m0);
      MOE_STAMPS_ONLY(st_x = stamp_clock(); if (m0 == 0) st_ph[10] += st_x - st_tile;)
      __syncthreads();
      for (int i = tid; i < 16 * MT; i += 256) fs[i] = i < nm ? perm[beg + m0 + i] : -1;
      if (MODE == 1 && tid < nsl) sg[tid] = sig[(int64_t)(beg + m0) * nsl + tid];
      __syncthreads();
      // activation rows of this pass (rows past the assignments repeat row 0)
      int64_t aoff[D::NAI];
      int apc[D::NAI];
#pragma unroll
      for (int i = 0; i < D::NAI; ++i) {
        const int row = (i * 4 + wave) * D::RPI + lane / D::SPR;
        const int fr = row < 16 * MT ? fs[row] : -1;
        const int f = fr >= 0 ? fr : fs[0];
        const int64_t src = MODE == 0 ? (int64_t)(f / k) : (int64_t)f;
        aoff[i] = src * K;
        apc[i] = 8 * ((lane % D::SPR) ^ D::swz_a(row));
      }
      float4v acc[MT][2];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[mt][c] = float4v{0.f, 0.f, 0.f, 0.f};

      auto issue = [&](int q, uint8_t* Bst) {
        uint8_t* Sst = Bst + D::B_BYTES;
        uint8_t* Ast = Sst + D::S_BYTES;
#pragma unroll
        for (int i = 0; i < D::NBI; ++i)
          dma16(Wexp + ro[i] + min(q * LB + bcol[i], rb - 16), Bst + (i * 4 + wave) * 1024);
#pragma unroll
        for (int i = 0; i < D::NSI; ++i)
          dma4(Sexp + so[i] + min(q * D::BPS + sp[i], NB - 2), Sst + (i * 4 + wave) * 256);
        // Activation rows past the pass's last assignment are only ever
        // multiplied into discarded output rows, so a wave whose rows all lie
        // there skips its load (the rows keep whatever the stage held). With a
        // two-stage ring every wait is for all loads in flight, so the skipped
        // loads do not upset the wait counts; deeper rings load every row
        // (replacing those loads with 4-byte ones, which count the same, was
        // measured slower).
#pragma unroll
        for (int i = 0; i < D::NAI; ++i) {
          if (NS == 2 && (i * 4 + wave) * D::RPI >= nm) continue;
          dma16(act + aoff[i] + min(q * D::KC + apc[i], K - 8), Ast + (i * 4 + wave) * 1024);
        }
      };
      // One stage: for each of its BPS blocks, the lane group's 8 codes of its
      // two rows become B fragments, each M tile's activation fragment of the
      // block is A, and every MFMA's fp32 partial is added times its row's
      // block scale. The next block's activation fragments are read while the
      // current block's MFMAs run.
      // NR: how many of a lane's four rows per tile take the scale FMAs (4 but
      // in one-tile passes of at most three assignments)
      auto compute = [&](int q, const uint8_t* Bst, auto NRc) {
        constexpr int NR = decltype(NRc)::value;
        uint32_t bb = lds_addr(Bst);
        // One-tile passes are bound by bytes in flight, so by occupancy: the
        // stage base is hidden from the optimiser, and each LDS address is
        // formed where it is used instead of being hoisted, for every unrolled
        // stage, into registers held across the loop.
        if constexpr (MT == 1) asm("" : "+v"(bb));
        const uint32_t sb = bb + D::B_BYTES;
        const uint32_t ab = sb + D::S_BYTES;
        CodeWords<SCHEME> cw0[D::BPS], cw1[D::BPS];
        typename D::ScaleWord sw[2];
        typename D::SigWord sgw[1];
#pragma unroll
        for (int b = 0; b < D::BPS; ++b) {
          lds_read(bb + lrow[0] * LB + D::code_off(lrow[0], b, g), cw0[b]);
          lds_read(bb + lrow[1] * LB + D::code_off(lrow[1], b, g), cw1[b]);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) lds_read(sb + lrow[c] * D::BPS * 2, sw[c]);
        if constexpr (MODE == 1) lds_read(lds_addr(sg) + (q * D::KC / 64) * 4, sgw[0]);
        auto read_a = [&](int b, u32x4 (&a)[MT]) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            lds_read(ab + (mt * 16 + r16) * D::ARB + (((4 * b + g) ^ D::swz_a(r16)) << 4), a[mt]);
        };
        u32x4 fa[2][MT];
        read_a(0, fa[0]);
        lds_wait(cw0);
        lds_wait(cw1);
        lds_wait(sw);
        if constexpr (MODE == 1) lds_wait(sgw);
        // a block's scales, zero past the row end (K tail) or for a slot-less
        // expert; the mask keeps this free of branches, which would split the
        // scheduling region of the MFMA chain
        const uint32_t live = resident ? 0xFFFFu : 0u;
        auto scale = [&](int c, int b) {
          uint32_t m = q * D::BPS + b < NB ? live : 0u;
          asm("" : "+v"(m));
          float v = f16_bits_to_f32((uint16_t)(scale_bits(sw[c], b) & m));
          // down: h of this block's 64-column slice was stored times 2^-sigma
          if constexpr (MODE == 1) v = ldexpf(v, word_at(sgw[0], b >> 1));
          // converted here, once per block: folded into each FMA instead
          // (v_fma_mix_f32 on the fp16 bits) the FMAs run slower
          asm("" : "+v"(v));
          return v;
        };
        typename M::v8 bc0 = codes8<SCHEME, AT>(cw0[0]), bc1 = codes8<SCHEME, AT>(cw1[0]);
        lds_wait(fa[0]);
#pragma unroll
        for (int b = 0; b < D::BPS; ++b) {
          const float s0 = scale(0, b), s1 = scale(1, b);
          if (b + 1 < D::BPS) read_a(b + 1, fa[(b + 1) & 1]);
          // Every M tile runs, also past the pass's last assignment (those rows
          // repeat a valid row and are discarded): no branches between the MFMAs.
          // The 2 MT products go out in a chain where product j is issued before
          // the four scale FMAs of product j-1, in two alternating registers, so
          // the FMAs (and the conversion of the next block's codes) run while the
          // next MFMA is in the matrix core instead of waiting for their own.
          typename M::v8 bn0, bn1;
          float4v pp[2];
          static_for<2 * MT>([&](auto J) {
            constexpr int j = decltype(J)::value;
            pp[j & 1] = M::run(a_operand<SCHEME, AT>(fa[b & 1][j / 2]), (j & 1) ? bc1 : bc0);
            if constexpr (j > 0)
              scaled_add_n<NR>(acc[(j - 1) / 2][(j - 1) & 1], ((j - 1) & 1) ? s1 : s0, pp[(j - 1) & 1]);
            if constexpr (j == 0) {
              if (b + 1 < D::BPS) {
                bn0 = codes8<SCHEME, AT>(cw0[b + 1]);
                bn1 = codes8<SCHEME, AT>(cw1[b + 1]);
              }
            }
            sched_group<kSchedMfma, 1>();
            sched_group<kSchedValu, j == 0 ? 2 : 2 + NR>();
          });
          scaled_add_n<NR>(acc[MT - 1][1], s1, pp[(2 * MT - 1) & 1]);
          if (b + 1 < D::BPS) {
            bc0 = bn0;
            bc1 = bn1;
            lds_wait(fa[(b + 1) & 1]);
          }
        }
      };

      // Every iteration issues one stage and waits for the oldest one, so all
      // waits are the same constant; past the last chunk a deeper ring refills a
      // stage with the last chunk again (clamped, cache-resident, never read) to
      // keep that count. A two-stage ring waits for everything in flight, so it
      // issues nothing past the last chunk.
      MOE_STAMPS_ONLY(const unsigned long long st_p = stamp_clock(); st_ph[5] += st_p - st_x;)
      static_for<NS - 1>([&](auto R) { issue(min((int)decltype(R)::value, nchunks - 1), stage(R)); });
      MOE_STAMPS_ONLY(st_ph[6] += stamp_clock() - st_p;)
      // chunk q lives in stage q % NS; the loop is unrolled NS times so that every
      // stage index is a constant
      auto k_loop = [&](auto NRc) {
      for (int q0 = 0; q0 < nchunks; q0 += NS) {
        static_for<NS>([&](auto R) {
          constexpr int r = decltype(R)::value;
          const int q = q0 + r;
          if (q < nchunks) {
            MOE_STAMPS_ONLY(const unsigned long long st_a = stamp_clock();)
            wait_vmcnt<(NS - 2) * D::NI>();
            MOE_STAMPS_ONLY(const unsigned long long st_b = stamp_clock();)
            raw_barrier();  // chunk q is in LDS for every wave; chunk q-1's stage is free
            MOE_STAMPS_ONLY(const unsigned long long st_c = stamp_clock();)
            if (NS > 2 || q + 1 < nchunks) issue(min(q + NS - 1, nchunks - 1), stage(ICg<(r + NS - 1) % NS>{}));
            compute(q, stage(R), NRc);  // ends with its LDS reads complete
            MOE_STAMPS_ONLY(st_ph[0] += st_b - st_a; st_ph[1] += st_c - st_b; st_ph[2] += stamp_clock() - st_c;)
          }
        });
      }
      };
      // A one-tile pass of nm <= 3 assignments keeps rows 0 .. nm-1, all in lane
      // group 0: only the first nm of a lane's four rows need the scale FMAs (a
      // uniform branch per pass, outside the MFMA chain). Batched decode passes
      // mostly hold one to three assignments. Gate/up only: the one-tile down
      // GEMM waits on its loads, and the larger code made it slower.
      if constexpr (MT == 1 && MODE == 0) {
        if (nm == 1) k_loop(ICg<1>{});
        else if (nm == 2) k_loop(ICg<2>{});
        else if (nm == 3) k_loop(ICg<3>{});
        else k_loop(ICg<4>{});
      } else {
        k_loop(ICg<4>{});
      }
      MOE_STAMPS_ONLY(const unsigned long long st_w = stamp_clock();)
      wait_vmcnt<0>();  // the trailing refills land before the next pass reuses the stages
      MOE_STAMPS_ONLY(st_x = stamp_clock(); st_ph[7] += st_x - st_w;)
      // epilogue: lane holds rows m = mt*16 + 4g + i of its two 16-column tiles, column r16.
      // A pass with all 16*MT rows and all of the workgroup's columns in range
      // (the common case in large batches) takes a form without the row and
      // column tests, which otherwise wrap every store in a branch.
      const bool full = nm == 16 * MT && n0 + (MODE == 0 ? 64 : 128) <= lim;
      if constexpr (MODE == 0) {
        // gate tile column n0 + 16*wave + r16 pairs with the same up tile column
        const int n = n0 + wave * 16 + r16;
        auto epilogue = [&](auto FULLc) {
          constexpr bool FULL = decltype(FULLc)::value;
          float hv[MT][4], amax = 0.0f;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              hv[mt][i] = silu(acc[mt][0][i]) * acc[mt][1][i];
              if (FULL || (mt * 16 + 4 * g + i < nm && n < lim)) amax = fmaxf(amax, fabsf(hv[mt][i]));
            }
          const int sigma = tile_sigma(workgroup_absmax(amax, red));
          if (tid == 0) sig[(int64_t)(beg + m0) * nsl + cb] = sigma;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = mt * 16 + 4 * g + i;
              if (FULL || (m < nm && n < lim))
                h16[(int64_t)fs[m] * I + n] = to_act16<MOE_F16>(ldexpf(hv[mt][i], -sigma));
            }
        };
        if (full) epilogue(std::true_type{});
        else epilogue(std::false_type{});
        MOE_STAMPS_ONLY(st_ph[8] += stamp_clock() - st_x;)
      } else if constexpr (!OHALF) {
        // fp32 rows
        auto epilogue = [&](auto FULLc) {
          constexpr bool FULL = decltype(FULLc)::value;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = mt * 16 + 4 * g + i;
              if (!FULL && m >= nm) continue;
              const int f = fs[m];
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                const int n = n0 + wave * 32 + 16 * c + r16;
                if (FULL || n < lim) ys[(int64_t)f * H + n] = acc[mt][c][i];
              }
            }
          }
        };
        if (full) epilogue(std::true_type{});
        else epilogue(std::false_type{});
        MOE_STAMPS_ONLY(st_ph[8] += stamp_clock() - st_x;)
      } else {
        // per-slot rows ahead of the combine, stored as h is: fp16 of
        // y * 2^-sigma, with the largest |y| of the wave's tile (the pass's
        // rows x its 32 columns) in [2^14, 2^15), and sigma for each of the
        // tile's rows at osig[f][n/32]
        const int nsl32 = (H + 31) / 32, sl32 = (n0 + wave * 32) / 32;
        auto epilogue = [&](auto FULLc) {
          constexpr bool FULL = decltype(FULLc)::value;
          float amax = 0.0f;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int c = 0; c < 2; ++c)
                if (FULL || (mt * 16 + 4 * g + i < nm && n0 + wave * 32 + 16 * c + r16 < lim))
                  amax = fmaxf(amax, fabsf(acc[mt][c][i]));
          const int sigma = tile_sigma(wave_max(amax));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = mt * 16 + 4 * g + i;
              if (!FULL && m >= nm) continue;
              const int f = fs[m];
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                const int n = n0 + wave * 32 + 16 * c + r16;
                if (FULL || n < lim) o16[(int64_t)f * H + n] = to_act16<MOE_F16>(ldexpf(acc[mt][c][i], -sigma));
              }
            }
          }
          return sigma;
        };
        const int sigma = full ? epilogue(std::true_type{}) : epilogue(std::false_type{});
        if (sl32 < nsl32)
          for (int m = lane; m < nm; m += 64) osig[(int64_t)fs[m] * nsl32 + sl32] = sigma;
        MOE_STAMPS_ONLY(st_ph[8] += stamp_clock() - st_x;)
      }
    }
    MOE_STAMPS_ONLY(st_ph[9] += stamp_clock() - st_tile;)
  }
  MOE_STAMPS_ONLY(st_ph[3] = stamp_clock() - st_t0; st_ph[4] = 1; if (lane == 0) {
    for (int i = 0; i < 11; ++i) atomicAdd(&g_stamps_gemm[MODE][i], st_ph[i]);
  })
}

// Workgroups of a kernel that fit on the device at once (a multiple of 8).
template <typename K>
static int resident_workgroups(K kernel) {
  int per_cu = 0, dev = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess || per_cu < 1) per_cu = 1;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  return (per_cu * cus + 7) / 8 * 8;
}

template <int SCHEME, int AT, int MODE, int MT, int NS, int LB, bool OHALF = false>
static void launch_dma(int ncb, int maxu8, const uint16_t* act, const ExpertsDev& ex, int k, const GroupBufs& g,
                       uint16_t* h16, int32_t* sig, float* ys, uint16_t* o16, int32_t* osig, hipStream_t s) {
  auto kernel = k_gemm_dma<SCHEME, AT, MODE, MT, NS, LB, OHALF>;
  static const int resident = resident_workgroups(kernel);  // per kernel, first call
  const int grid = std::min(resident, ncb * maxu8);
  MOE_LAUNCH(MODE == 0 ? MOE_KERNEL_GEMM_GATE_UP : MOE_KERNEL_GEMM_DOWN, kernel, dim3(grid), dim3(256), 0, s, act,
             ex, k, g.uniq, g.n_uniq, g.counts, g.offsets, g.perm, h16, sig, ys, o16, osig, ncb);
}

// gate/up (activations of type AT) then down (fp16 h), with one tuning: M
// tiles per pass, stages, line bytes per stage. Both take the same passes, so
// the down GEMM finds the tile exponents of h where gate/up left them. The
// down GEMM writes fp32 rows to out, or (out null) fp16 rows with their tile
// exponents to o16 / osig.
template <int SCHEME, int AT, int MT, int NS, int LB, int LBD = LB>
static void launch_dma_pair(int maxu8, const uint16_t* x, const ExpertsDev& ex, int k, const GroupBufs& g,
                            uint16_t* h16, int32_t* sig, float* out, uint16_t* o16, int32_t* osig, hipStream_t s) {
  launch_dma<SCHEME, AT, 0, MT, NS, LB>((ex.I + 63) / 64, maxu8, x, ex, k, g, h16, sig, nullptr, nullptr, nullptr, s);
  if (o16)
    launch_dma<SCHEME, MOE_F16, 1, MT, NS, LBD, true>((ex.H + 127) / 128, maxu8, h16, ex, k, g, h16, sig, nullptr, o16,
                                                      osig, s);
  else
    launch_dma<SCHEME, MOE_F16, 1, MT, NS, LBD>((ex.H + 127) / 128, maxu8, h16, ex, k, g, h16, sig, out, nullptr,
                                                nullptr, s);
}

hipError_t launch_gemm_grouped(const void* x, int xtype, int T, const ExpertsDev& ex, int k, const GroupBufs& g,
                               const float* gate, uint16_t* h16, int32_t* sig, float* ys, float* y, hipStream_t s) {
  if (xtype != MOE_F16 && xtype != MOE_BF16) return hipErrorInvalidValue;  // callers route fp32 elsewhere
  const int maxu = (int)std::min<int64_t>((int64_t)ex.E, (int64_t)T * k);
  const double avg = (double)T * k / ex.E;
  // down output: the per-slot rows ahead of the combine, or the caller's
  // per-slot output (fp32) when no gates are given ([T][k][H] in both cases).
  // Where fp32 rows ahead of the combine would not fit the 256 MB last-level
  // cache, the DMA kernel stores fp16 rows with a power of two per 32 columns
  // instead, in the fp32 rows' space: the rows first (half of it), then their
  // exponents, [T*k][H/32]. That halves the rows' write and read traffic
  // (measured 1137 -> 1094 us per layer at 8192 tokens); smaller batches keep
  // fp32 rows, whose traffic is cheaper than the exponents' epilogue.
  float* out = gate ? ys : y;
  uint16_t* ys16 = reinterpret_cast<uint16_t*>(ys);
  int32_t* ysig = reinterpret_cast<int32_t*>(ys16 + (int64_t)T * k * ex.H);
  bool half_rows = false;
  const uint16_t* act = static_cast<const uint16_t*>(x);
  auto with_at = [&](auto ATc) {
    constexpr int AT = decltype(ATc)::value;
    if (ex.H % 64 == 0 && ex.I % 64 == 0) {
      const int maxu8 = (maxu + 7) / 8 * 8;
      // Tunings measured on MI355X. Whole 128-byte lines per stage with two
      // stages keep three workgroups per CU for one- and four-tile passes;
      // six-tile passes (about 64 assignments per expert and more) stage half
      // lines in three stages. int4 four-tile passes use half lines.
      half_rows = gate != nullptr && (int64_t)T * k * ex.H * 4 > ((int64_t)256 << 20);
      float* o32 = half_rows ? nullptr : out;
      uint16_t* o16 = half_rows ? ys16 : nullptr;
      int32_t* osig = half_rows ? ysig : nullptr;
      if (ex.scheme == MOE_Q_SYM8) {
        if (avg > 24) launch_dma_pair<MOE_Q_SYM8, AT, 6, 3, 64>(maxu8, act, ex, k, g, h16, sig, o32, o16, osig, s);
        else if (avg > 6) launch_dma_pair<MOE_Q_SYM8, AT, 4, 2, 128>(maxu8, act, ex, k, g, h16, sig, o32, o16, osig, s);
        else launch_dma_pair<MOE_Q_SYM8, AT, 1, 2, 128>(maxu8, act, ex, k, g, h16, sig, o32, o16, osig, s);
      } else {
        if (avg > 6) launch_dma_pair<MOE_Q_INT4, AT, 4, 2, 64>(maxu8, act, ex, k, g, h16, sig, o32, o16, osig, s);
        else launch_dma_pair<MOE_Q_INT4, AT, 1, 2, 128, 64>(maxu8, act, ex, k, g, h16, sig, o32, o16, osig, s);
      }
      return;
    }
    // rows with an odd number of 32-element blocks: the register-staged kernel
    auto run = [&](auto SC, auto MTc) {
      constexpr int S_ = decltype(SC)::value, MT_ = decltype(MTc)::value;
      dim3 g1((ex.I + 63) / 64, maxu), g2((ex.H + 127) / 128, maxu);
      MOE_LAUNCH(MOE_KERNEL_GEMM_GATE_UP, (k_gemm_grouped<S_, AT, 0, MT_>), g1, dim3(256), 0, s, act, ex, k, g.uniq,
                 g.n_uniq, g.counts, g.offsets, g.perm, h16, sig, static_cast<float*>(nullptr));
      MOE_LAUNCH(MOE_KERNEL_GEMM_DOWN, (k_gemm_grouped<S_, MOE_F16, 1, MT_>), g2, dim3(256), 0, s,
                 static_cast<const uint16_t*>(h16), ex, k, g.uniq, g.n_uniq, g.counts, g.offsets, g.perm, h16, sig,
                 out);
    };
    auto with_mt = [&](auto SC) {
      if (avg > 24) run(SC, ICg<8>{});
      else if (avg > 6) run(SC, ICg<4>{});
      else run(SC, ICg<1>{});
    };
    if (ex.scheme == MOE_Q_SYM8) with_mt(ICg<MOE_Q_SYM8>{});
    else with_mt(ICg<MOE_Q_INT4>{});
  };
  if (xtype == MOE_F16) with_at(ICg<MOE_F16>{});
  else with_at(ICg<MOE_BF16>{});
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (gate) return half_rows ? launch_combine(T, ex.H, k, gate, nullptr, ys16, ysig, y, s)
                             : launch_combine(T, ex.H, k, gate, ys, nullptr, nullptr, y, s);
  return hipSuccess;
}

}  // namespace moe

#ifdef MOE_STAMPS
MOE_STAMP_READER(moe_stamps_read_gemm, moe::g_stamps_gemm)
extern "C" int moe_stamps_zero_gemm(void) {
  static const unsigned long long zero[2][16] = {};
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(moe::g_stamps_gemm), zero, sizeof(zero));
}
#endif
