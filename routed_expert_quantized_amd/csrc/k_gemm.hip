// k_gemm.hip — grouped MFMA GEMM for batched tokens (prefill and batched decode).
//
// After the token-by-expert grouping each routed expert e has n_e assignments.
// GEMM1: U_e[n_e][2I] = X_e[n_e][H] . W_gu[e]^T, then h = silu(gate) * up
//        (gate columns n and up columns I + n in the same workgroup), stored fp16.
// GEMM2: Y_e[n_e][H] = h_e[n_e][I] . W_d[e]^T, stored per assignment (ys): fp16
//        (round to nearest even) ahead of the combine, fp32 when it is the output.
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
#include <utility>

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
//   owns 128 rows; output ys16[f][n] (fp16) when ys16 is set, else ys[f][n] (fp32).
// The expert's assignments are taken 16*MT at a time (one pass each).
template <int SCHEME, int XT, int MODE, int MT>
__global__ __launch_bounds__(256) void k_gemm_grouped(const void* __restrict__ act, ExpertsDev ex, int k,
                                                      const int32_t* __restrict__ uniq,
                                                      const int32_t* __restrict__ n_uniq,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ perm, uint16_t* __restrict__ h16,
                                                      float* __restrict__ ys, uint16_t* __restrict__ ys16) {
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
            if (n < lim) {
              if (ys16) ys16[(int64_t)f * H + n] = __builtin_bit_cast(uint16_t, (_Float16)acc[mt][c][i]);
              else ys[(int64_t)f * H + n] = acc[mt][c][i];
            }
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
// for one 128-byte line of each of the workgroup's 128 weight rows: the codes
// (16 KiB), their fp16 block scales, and the 16*MT x KC fp16 activation tile.
// Activations come from fp16 rows (the input itself, a converted copy of it,
// or h). Scales move as 4-byte pairs, so a row must hold an even number of
// 32-element blocks (K a multiple of 64).
//
// Bank layout: a 16-byte LDS slot of code row r holds piece slot ^ ((r/2) & 7);
// of activation row r, piece slot ^ (r & 15). The DMA lane that fills a slot
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
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

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
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ uint32_t lds_read_u16(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_u16 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x4 (&a)[N]) {
  static_assert(N >= 1 && N <= 8, "fragment count");
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
__device__ __forceinline__ void lds_wait_b(u32x4 (&b)[4], uint32_t (&sc)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(sc[0]), "+v"(sc[1]), "+v"(sc[2]), "+v"(sc[3]));
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

// 8 fp16 weights (code * scale, one rounding) for MFMA step j of a lane's code
// span: sym8 words 2j and 2j+1; int4 word j, with the pairs in (c, c+4) order.
template <int SCHEME, int NW>
__device__ __forceinline__ half8v span_slice_f16(const uint32_t (&w)[NW], int j, half2v s2) {
  half8v r;
  if constexpr (SCHEME == MOE_Q_SYM8) {
    const half2v bias = as_h2(0xE480E480u);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t u = w[2 * j + t] ^ 0x80808080u;
      const half2v lo = (as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) + bias) * s2;
      const half2v hi = (as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) + bias) * s2;
      r[4 * t + 0] = lo[0]; r[4 * t + 1] = lo[1]; r[4 * t + 2] = hi[0]; r[4 * t + 3] = hi[1];
    }
  } else {
    const half2v bias = as_h2(0xE408E408u);
    const uint32_t u = w[j] ^ 0x88888888u;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const half2v v = (as_h2(((u >> (4 * p)) & 0x000F000Fu) | 0x64006400u) + bias) * s2;
      r[2 * p] = v[0];
      r[2 * p + 1] = v[1];
    }
  }
  return r;
}

// Stage geometry. LB bytes of each of the 128 weight rows per stage (64 or
// 128: half or whole cache lines); the four lane groups of a wave split them.
template <int SCHEME, int MT, int LB>
struct DmaTile {
  static constexpr int BB = SCHEME == MOE_Q_INT4 ? 16 : 32;  // bytes per 32-element block
  static constexpr int BPS = LB / BB;                        // blocks per row per stage
  static constexpr int KC = 32 * BPS;                        // K per stage
  static constexpr int NJ = KC / 32;                         // MFMA steps per stage
  static constexpr int SPAN = KC / 4;                        // K elements per lane group
  static constexpr int NW = LB / 16;                         // code words per lane group
  static constexpr int NSL = LB / 64;                        // 16-byte code slots per lane group
  static constexpr int NSC = SPAN >= 32 ? SPAN / 32 : 1;     // scales per lane group
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
  // slot swizzles: 16 lanes reading one logical slot of 16 consecutive rows hit
  // 16 distinct 16-byte bank groups
  static __device__ __forceinline__ int swz_b(int row) { return LB == 128 ? (row >> 1) & 7 : (row >> 2) & 3; }
  static __device__ __forceinline__ int swz_a(int row) { return SPR == 8 ? (row >> 1) & 7 : row & 15; }
};

// Waves per SIMD the register allocation must leave room for.
template <int SCHEME, int MT>
__host__ __device__ constexpr int gemm_dma_waves() {
  return 1;
}

template <int SCHEME, int MODE, int MT, int NS, int LB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(gemm_dma_waves<SCHEME, MT>(), 8)))
void k_gemm_dma(const uint16_t* __restrict__ act, ExpertsDev ex, int k,
                                                  const int32_t* __restrict__ uniq,
                                                  const int32_t* __restrict__ n_uniq,
                                                  const int32_t* __restrict__ counts,
                                                  const int32_t* __restrict__ offsets,
                                                  const int32_t* __restrict__ perm, uint16_t* __restrict__ h16,
                                                  float* __restrict__ ys, uint16_t* __restrict__ ys16, int ncb) {
  using D = DmaTile<SCHEME, MT, LB>;
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
  // Persistent: the grid holds as many workgroups as fit on the chip at once
  // (a multiple of 8), each taking tiles blockIdx.x, +gridDim.x, ... until the
  // routed experts' tiles run out, so no partly filled last round of
  // workgroups is left. Tile order is XCD-aware: ids go round-robin over the 8
  // XCDs, and tile (expert u, column block cb) has id (u/8)*8*ncb + cb*8 + u%8,
  // so all column blocks of an expert (which read the same activation rows)
  // run on one XCD, with the experts alternating over the XCDs.
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
    const int e = uniq[u], cnt = counts[e], beg = offsets[e];
    const int H = ex.H, I = ex.I;
    const int K = MODE == 0 ? H : I;
    const int NB = K / 32;
    const int NROW = MODE == 0 ? 2 * I : H;
    const int lim = MODE == 0 ? I : H;
    const int rb = (int)row_bytes<SCHEME>(K);
    const uint8_t* Wexp = (MODE == 0 ? ex.wgu : ex.wd) + (int64_t)e * NROW * rb;
    const uint16_t* Sexp = (MODE == 0 ? ex.sgu : ex.sd) + (int64_t)e * NROW * NB;
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

    // DMA sources that stay fixed for the whole kernel: code rows and scale rows
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

    for (int m0 = 0; m0 < cnt; m0 += 16 * MT) {
      const int nm = min(16 * MT, cnt - m0);
      __syncthreads();
      for (int i = tid; i < 16 * MT; i += 256) fs[i] = i < nm ? perm[beg + m0 + i] : -1;
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
      const int mtiles = (nm + 15) / 16;

      auto issue = [&](int q, uint8_t* Bst) {
        uint8_t* Sst = Bst + D::B_BYTES;
        uint8_t* Ast = Sst + D::S_BYTES;
  #pragma unroll
        for (int i = 0; i < D::NBI; ++i)
          dma16(Wexp + ro[i] + min(q * LB + bcol[i], rb - 16), Bst + (i * 4 + wave) * 1024);
  #pragma unroll
        for (int i = 0; i < D::NSI; ++i)
          dma4(Sexp + so[i] + min(q * D::BPS + sp[i], NB - 2), Sst + (i * 4 + wave) * 256);
  #pragma unroll
        for (int i = 0; i < D::NAI; ++i)
          dma16(act + aoff[i] + min(q * D::KC + apc[i], K - 8), Ast + (i * 4 + wave) * 1024);
      };
      auto compute = [&](int q, const uint8_t* Bst) {
        const uint32_t bb = lds_addr(Bst);
        const uint32_t sb = bb + D::B_BYTES;
        const uint32_t ab = sb + D::S_BYTES;
        // codes: lane group g's span of each of its two rows; scales of that span
        u32x4 raw[4] = {};
        uint32_t sc[4] = {0u, 0u, 0u, 0u};
  #pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int lr = lrow[c];
  #pragma unroll
          for (int t = 0; t < D::NSL; ++t)
            raw[2 * c + t] = lds_read16(bb + lr * LB + ((g * D::NSL + t) ^ D::swz_b(lr)) * 16);
  #pragma unroll
          for (int b = 0; b < D::NSC; ++b)
            sc[2 * c + b] = lds_read_u16(sb + (lr * D::BPS + g * D::SPAN / 32 + b) * 2);
        }
        // activation fragments of MFMA step j, M tiles mt0 .. mt0+G-1: row mt*16 + r16,
      // logical slot g*SPAN/8 + j. Steps go (j, group) in order; the next
      // group's fragments are read while the current group's MFMAs run.
      constexpr int G = MT % 4 == 0 ? 4 : MT % 3 == 0 ? 3 : MT % 2 == 0 ? 2 : 1;
      constexpr int NG = MT / G;
      auto read_a = [&](int j, int grp, u32x4 (&a)[G]) {
#pragma unroll
        for (int i = 0; i < G; ++i)
          a[i] = lds_read16(ab + ((grp * G + i) * 16 + r16) * D::ARB + (((g * D::SPAN / 8 + j) ^ D::swz_a(r16)) * 16));
      };
      u32x4 fa[2][G];
      read_a(0, 0, fa[0]);
      lds_wait_b(raw, sc);
      lds_wait<G>(fa[0]);
      uint32_t w[2][D::NW];
      half2v s2[2][D::NSC];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int t = 0; t < D::NSL; ++t) {
          const u32x4 v = raw[2 * c + t];
          w[c][4 * t + 0] = v.x; w[c][4 * t + 1] = v.y; w[c][4 * t + 2] = v.z; w[c][4 * t + 3] = v.w;
        }
#pragma unroll
        for (int b = 0; b < D::NSC; ++b) {
          // blocks past the row end (K tail) were clamped to valid memory; scale 0 drops them
          const float sv =
              q * D::BPS + g * D::SPAN / 32 + b < NB ? f16_bits_to_f32((uint16_t)sc[2 * c + b]) : 0.0f;
          s2[c][b] = half2v{(_Float16)sv, (_Float16)sv};
        }
      }
      half8v b[2];
#pragma unroll
      for (int st = 0; st < D::NJ * NG; ++st) {
        const int j = st / NG, grp = st % NG;
        if (grp == 0) {
#pragma unroll
          for (int c = 0; c < 2; ++c) b[c] = span_slice_f16<SCHEME, D::NW>(w[c], j, s2[c][j / 4]);
        }
        if (st + 1 < D::NJ * NG) read_a((st + 1) / NG, (st + 1) % NG, fa[(st + 1) & 1]);
#pragma unroll
        for (int i = 0; i < G; ++i) {
          if (grp * G + i < mtiles) {
            const u32x4 f = fa[st & 1][i];
            const half8v a = __builtin_bit_cast(half8v, order_for_b<SCHEME>(make_uint4(f.x, f.y, f.z, f.w)));
#pragma unroll
            for (int c = 0; c < 2; ++c)
              acc[grp * G + i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[c], acc[grp * G + i][c], 0, 0, 0);
          }
        }
        if (st + 1 < D::NJ * NG) lds_wait<G>(fa[(st + 1) & 1]);
      }
    };

    // Every iteration issues one stage and waits for the oldest one, so all
      // waits are the same constant; past the last chunk a stage is refilled with
      // the last chunk again (clamped, cache-resident) and never read.
      static_for<NS - 1>([&](auto R) { issue(min((int)decltype(R)::value, nchunks - 1), stage(R)); });
      // chunk q lives in stage q % NS; the loop is unrolled NS times so that every
      // stage index is a constant
      for (int q0 = 0; q0 < nchunks; q0 += NS) {
        static_for<NS>([&](auto R) {
          constexpr int r = decltype(R)::value;
          const int q = q0 + r;
          if (q < nchunks) {
            wait_vmcnt<(NS - 2) * D::NI>();
            raw_barrier();  // chunk q is in LDS for every wave; chunk q-1's stage is free
            issue(min(q + NS - 1, nchunks - 1), stage(ICg<(r + NS - 1) % NS>{}));
            compute(q, stage(R));  // ends with its LDS reads complete
          }
        });
      }
      wait_vmcnt<0>();  // the trailing refills land before the next pass reuses the stages
      // epilogue: lane holds rows m = mt*16 + 4g + i of its two 16-column tiles, column r16
  #pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mt * 16 + 4 * g + i;
          if (m >= nm) continue;
          const int f = fs[m];
          if (MODE == 0) {
            // gate tile column n0 + 16*wave + r16 pairs with the same up tile column
            const int n = n0 + wave * 16 + r16;
            if (n < lim) {
              const float hv = silu(acc[mt][0][i]) * acc[mt][1][i];
              h16[(int64_t)f * I + n] = __builtin_bit_cast(uint16_t, (_Float16)hv);
            }
          } else {
  #pragma unroll
            for (int c = 0; c < 2; ++c) {
              const int n = n0 + wave * 32 + 16 * c + r16;
              if (n < lim) {
                if (ys16) ys16[(int64_t)f * H + n] = __builtin_bit_cast(uint16_t, (_Float16)acc[mt][c][i]);
                else ys[(int64_t)f * H + n] = acc[mt][c][i];
              }
            }
          }
        }
      }
    }
  }
}

// fp16 copy of the activations (round to nearest even), for the DMA path's
// activation tiles: n8 groups of 8 elements.
template <int XT>
__global__ __launch_bounds__(256) void k_to_f16(const void* __restrict__ x, int64_t n8, uint16_t* __restrict__ out) {
  constexpr int xb = XT == MOE_F32 ? 4 : 2;
  const uint8_t* xs = static_cast<const uint8_t*>(x);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride)
    *reinterpret_cast<uint4*>(out + 8 * i) = load8_f16<XT>(xs + 8 * xb * i, 0);
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

template <int SCHEME, int MODE, int MT, int NS, int LB>
static void launch_dma(int ncb, int maxu8, const uint16_t* act, const ExpertsDev& ex, int k, const GroupBufs& g,
                       uint16_t* h16, float* ys, uint16_t* ys16, hipStream_t s) {
  auto kernel = k_gemm_dma<SCHEME, MODE, MT, NS, LB>;
  static const int resident = resident_workgroups(kernel);  // per kernel, first call
  const int grid = std::min(resident, ncb * maxu8);
  MOE_LAUNCH(MODE == 0 ? MOE_KERNEL_GEMM_GATE_UP : MOE_KERNEL_GEMM_DOWN, kernel, dim3(grid), dim3(256), 0, s, act,
             ex, k, g.uniq, g.n_uniq, g.counts, g.offsets, g.perm, h16, ys, ys16, ncb);
}

// gate/up then down with one tuning (M tiles per pass, stages, line bytes per stage)
template <int SCHEME, int MT, int NS, int LB>
static void launch_dma_pair(int maxu8, const uint16_t* act, const ExpertsDev& ex, int k, const GroupBufs& g,
                            uint16_t* h16, float* out, uint16_t* out16, hipStream_t s) {
  launch_dma<SCHEME, 0, MT, NS, LB>((ex.I + 63) / 64, maxu8, act, ex, k, g, h16, nullptr, nullptr, s);
  launch_dma<SCHEME, 1, MT, NS, LB>((ex.H + 127) / 128, maxu8, h16, ex, k, g, h16, out, out16, s);
}

hipError_t launch_gemm_grouped(const void* x, int xtype, int T, const ExpertsDev& ex, int k, const GroupBufs& g,
                               const float* gate, uint16_t* h16, uint16_t* x16, float* ys, float* y, hipStream_t s) {
  const int maxu = (int)std::min<int64_t>((int64_t)ex.E, (int64_t)T * k);
  const double avg = (double)T * k / ex.E;
  // down output: fp16 per-slot rows ahead of the combine, or the caller's
  // fp32 per-slot output when no gates are given
  float* out = gate ? nullptr : y;
  uint16_t* out16 = gate ? reinterpret_cast<uint16_t*>(ys) : nullptr;
  if (ex.H % 64 == 0 && ex.I % 64 == 0) {
    // activations as fp16 rows
    const uint16_t* act = static_cast<const uint16_t*>(x);
    if (xtype != MOE_F16) {
      const int64_t n8 = (int64_t)T * ex.H / 8;
      const int blocks = (int)std::min<int64_t>((n8 + 255) / 256, 4096);
      if (xtype == MOE_F32)
        hipLaunchKernelGGL(k_to_f16<MOE_F32>, dim3(blocks), dim3(256), 0, s, x, n8, x16);
      else
        hipLaunchKernelGGL(k_to_f16<MOE_BF16>, dim3(blocks), dim3(256), 0, s, x, n8, x16);
      act = x16;
    }
    const int maxu8 = (maxu + 7) / 8 * 8;
    // Tunings measured on MI355X. Whole 128-byte lines per stage with two stages
    // keep three workgroups per CU for one- and four-tile passes; six-tile passes
    // (about 64 assignments per expert and more) stage half lines in three
    // stages (taller passes measured no faster at ~256 assignments per expert).
    // int4 four-tile passes use half lines (whole lines exceed the registers).
    if (ex.scheme == MOE_Q_SYM8) {
      if (avg > 24) launch_dma_pair<MOE_Q_SYM8, 6, 3, 64>(maxu8, act, ex, k, g, h16, out, out16, s);
      else if (avg > 6) launch_dma_pair<MOE_Q_SYM8, 4, 2, 128>(maxu8, act, ex, k, g, h16, out, out16, s);
      else launch_dma_pair<MOE_Q_SYM8, 1, 2, 128>(maxu8, act, ex, k, g, h16, out, out16, s);
    } else {
      if (avg > 6) launch_dma_pair<MOE_Q_INT4, 4, 2, 64>(maxu8, act, ex, k, g, h16, out, out16, s);
      else launch_dma_pair<MOE_Q_INT4, 1, 2, 128>(maxu8, act, ex, k, g, h16, out, out16, s);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (gate) return launch_combine(T, ex.H, k, gate, nullptr, out16, y, s);
    return hipGetLastError();
  }
  // rows with an odd number of 32-element blocks: register-staged kernel
  auto run = [&](auto SC, auto XC, auto MTc) {
    constexpr int S_ = decltype(SC)::value, X_ = decltype(XC)::value, MT_ = decltype(MTc)::value;
    dim3 g1((ex.I + 63) / 64, maxu), g2((ex.H + 127) / 128, maxu);
    MOE_LAUNCH(MOE_KERNEL_GEMM_GATE_UP, (k_gemm_grouped<S_, X_, 0, MT_>), g1, dim3(256), 0, s, x, ex, k, g.uniq,
               g.n_uniq, g.counts, g.offsets, g.perm, h16, static_cast<float*>(nullptr),
               static_cast<uint16_t*>(nullptr));
    MOE_LAUNCH(MOE_KERNEL_GEMM_DOWN, (k_gemm_grouped<S_, MOE_F16, 1, MT_>), g2, dim3(256), 0, s,
               (const void*)h16, ex, k, g.uniq, g.n_uniq, g.counts, g.offsets, g.perm, h16, out, out16);
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
  if (gate) return launch_combine(T, ex.H, k, gate, nullptr, out16, y, s);
  return hipGetLastError();
}

}  // namespace moe
