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
#include <algorithm>
#include <type_traits>

#include "head_rows.hpp"
#include "kernels.hpp"
#include "stamps.hpp"

namespace moe {

// timestamp build only. Single-token gate/up workgroups: 0 start, 1 routing
// known, 2 weight loads landed, 3 end; down workgroups: 4 start, 5 routing
// read, 6 weight loads landed, 7 end.
MOE_STAMP_TABLE(g_stamps_decode, 8);

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


// ------------------------------------------------------------------ T = 1
// Waves per workgroup of the single-token gate/up kernel (each owns one row pair).
constexpr int kGateUpWaves = 4;

// Grid: k slots x blocks_per_slot (+1 from logits). A wave computes RP (gate
// row n, up row I+n) pairs of its slot's expert and writes h[slot][n] =
// silu(gate) * up. ROUTE 0: the routing is given (idx_in, expert ids, mapped
// through the slot table when there is one). ROUTE 1: wave 0 of each
// workgroup first picks the top k from the router logits, as far as its slot
// (every workgroup redoes this small step, so no cross-workgroup sync is
// needed); one extra workgroup publishes the routing for the down kernel and
// the caller. ROUTE 2: as 1, with each pick's slot-table entry (the expert's
// slot in a resident stack) as the weights' index.
// With H16 the activation is stored as fp16 (round to nearest even) for the
// slot-parallel down kernel, else as fp32.
template <int SCHEME, int XT, int NBJ, int RP, int ROUTE, int VPL, bool H16>
__device__ __forceinline__ void gate_up_t1_body(const void* __restrict__ x, const ExpertsDev& ex, int k, int renorm,
                                                const float* __restrict__ logits,
                                                const int32_t* __restrict__ idx_in,
                                                int32_t* __restrict__ idx_ws, float* __restrict__ gate_ws,
                                                int32_t* __restrict__ idx_user, float* __restrict__ gate_user,
                                                float* __restrict__ h, int blocks_per_slot, int bid) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slot = bid / blocks_per_slot, blk = bid % blocks_per_slot;
  const int H = ex.H, I = ex.I, NB = H / 32;
  MOE_STAMP(g_stamps_decode, 0, bid);
  // Every load below is unconditional (block and row indices are clamped in
  // bounds, surplus lanes get a zero scale) so the scheduler can issue them all
  // before the arithmetic.
  // Activations do not depend on the routing: they are requested first, into
  // registers, and stay in flight while the routing's logits are read. fp16
  // activations with the routing step then go through LDS, one 16-byte piece
  // per thread, behind the barriers that share the routing (one read of x per
  // workgroup instead of one per wave); otherwise each wave loads its blocks.
  constexpr bool FROM_LOGITS = ROUTE != 0;
  constexpr bool kStageX = XT == MOE_F16 && FROM_LOGITS;
  constexpr int kThreads = 64 * kGateUpWaves;
  constexpr int kXPieces = kStageX ? (NBJ * 256 + kThreads - 1) / kThreads : 1;
  __shared__ uint4 xs[kStageX ? NBJ * 256 : 1];
  XReg<SCHEME, XT> xr[NBJ];
  uint4 xv[kXPieces];
  if constexpr (kStageX) {
#pragma unroll
    for (int j = 0; j < kXPieces; ++j)
      xv[j] = reinterpret_cast<const uint4*>(x)[min((int)threadIdx.x + kThreads * j, H / 8 - 1)];
  } else {
#pragma unroll
    for (int j = 0; j < NBJ; ++j) load_xreg<SCHEME, XT>(xr[j], x, 0, min(lane + 64 * j, NB - 1));
  }
  int e;
  if constexpr (FROM_LOGITS) {
    // One extra workgroup, after the k slots' ones, publishes the routing for
    // the down kernel and the caller: it ranks all k experts and computes
    // their gates (lane s < k of its wave 0 holds rank s) and reads no
    // weights, so no weight-reading workgroup waits for the gates.
    if (bid == k * blocks_per_slot) {
      if (wave == 0) {
        int my_idx, my_row;
        float my_gate;
        if constexpr (ROUTE == 2) {
          wave_topk<VPL, true>(logits, ex.E, k, renorm != 0, my_idx, my_gate, k, ex.slot_of, ex.slots, &my_row);
        } else {
          wave_topk<VPL>(logits, ex.E, k, renorm != 0, my_idx, my_gate, k);
          my_row = my_idx;
        }
        // the down kernel reads the weights' indices (slots when staged), the caller the expert ids
        if (lane < k) {
          idx_ws[lane] = my_row;
          gate_ws[lane] = my_gate;
          if (idx_user) idx_user[lane] = my_idx;
          if (gate_user) gate_user[lane] = my_gate;
        }
      }
      return;
    }
    // A workgroup of slot s needs only the first s+1 rounds. Wave 0 picks the
    // routing (with a slot table, each rank's entry comes along); the other
    // waves store the activations and wait for it at the barrier.
    __shared__ int e_sh;
    if (wave == 0) {
      int my_idx, my_row;
      float my_gate;
      if constexpr (ROUTE == 2) {
        wave_topk<VPL, true>(logits, ex.E, k, renorm != 0, my_idx, my_gate, slot + 1, ex.slot_of, ex.slots, &my_row);
      } else {
        wave_topk<VPL>(logits, ex.E, k, renorm != 0, my_idx, my_gate, slot + 1);
        my_row = my_idx;
      }
      if (lane == slot) e_sh = my_row;
    }
    if constexpr (kStageX) {
#pragma unroll
      for (int j = 0; j < kXPieces; ++j) {
        const int i = (int)threadIdx.x + kThreads * j;
        if (i < H / 8) xs[i] = xv[j];
      }
    }
    __syncthreads();
    e = e_sh;
    MOE_STAMP(g_stamps_decode, 1, bid);
  } else {
    e = expert_index(ex, idx_in[slot]);
  }
  // an expert without a slot contributes nothing: index 0 is read with zero scales
  const bool resident = e >= 0;  // a slot-less expert: zero scales, whatever slot 0 holds
  e = max(e, 0);
  if constexpr (kStageX) {
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      const int b = min(lane + 64 * j, NB - 1);
      uint32_t nat[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = xs[4 * b + i];
        nat[4 * i] = v.x; nat[4 * i + 1] = v.y; nat[4 * i + 2] = v.z; nat[4 * i + 3] = v.w;
      }
      xr[j].h = xblock_from_pairs<SCHEME>(nat);
    }
  }
  const int n0 = (blk * kGateUpWaves + wave) * RP;
  const int64_t rb = row_bytes<SCHEME>(H);
  Block<SCHEME> cg[RP][NBJ], cu[RP][NBJ];
  float sg[RP][NBJ], su[RP][NBJ];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int n = min(n0 + r, I - 1);  // rows past I are read in bounds and discarded
    const int64_t grow = (int64_t)e * 2 * I + n, urow = grow + I;
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      const int b = min(lane + 64 * j, NB - 1);
      cg[r][j] = load_block<SCHEME>(ex.wgu + grow * rb, b);
      cu[r][j] = load_block<SCHEME>(ex.wgu + urow * rb, b);
      sg[r][j] = scale_or_zero(ex.sgu + grow * NB + b, resident);
      su[r][j] = scale_or_zero(ex.sgu + urow * NB + b, resident);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  MOE_STAMP_LANDED(g_stamps_decode, 2, bid);
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    float ag = 0.0f, au = 0.0f;
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      const bool valid = lane + 64 * j < NB;
      ag = fmaf(valid ? sg[r][j] : 0.0f, xdot<SCHEME, XT>(cg[r][j], xr[j]), ag);
      au = fmaf(valid ? su[r][j] : 0.0f, xdot<SCHEME, XT>(cu[r][j], xr[j]), au);
    }
    ag = wave_sum(ag);
    au = wave_sum(au);
    if (lane == 0 && n0 + r < I) {
      const float hv = silu(ag) * au;
      if constexpr (H16) reinterpret_cast<uint16_t*>(h)[(int64_t)slot * I + n0 + r] = __builtin_bit_cast(uint16_t, (_Float16)hv);
      else h[(int64_t)slot * I + n0 + r] = hv;
    }
  }
  MOE_STAMP(g_stamps_decode, 3, bid);
}

template <int SCHEME, int XT, int NBJ, int RP, int ROUTE, int VPL, bool H16>
__global__ __launch_bounds__(64 * kGateUpWaves) void k_gate_up_t1(const void* __restrict__ x, ExpertsDev ex, int k, int renorm,
                                                    const float* __restrict__ logits,
                                                    const int32_t* __restrict__ idx_in,
                                                    int32_t* __restrict__ idx_ws, float* __restrict__ gate_ws,
                                                    int32_t* __restrict__ idx_user, float* __restrict__ gate_user,
                                                    float* __restrict__ h, int blocks_per_slot) {
  gate_up_t1_body<SCHEME, XT, NBJ, RP, ROUTE, VPL, H16>(x, ex, k, renorm, logits, idx_in, idx_ws, gate_ws,
                                                             idx_user, gate_user, h, blocks_per_slot, blockIdx.x);
}

// Single-token down, one wave per slot. Grid: ceil(H / (4 RW)) workgroups of
// k waves. Wave q takes slot q; its four 16-lane row groups take RW rows each,
// and lane ll of a group owns blocks ll + 16 j of the I inputs for those rows,
// so the fp16 h block it loads once serves all RW rows. Row sums over the 16
// lanes are kept in LDS; after a barrier the first 4 RW threads add the slots in
// slot order, each times its gate (with gate == nullptr every wave writes its
// own slot's rows, y[q][m]). Many small waves per CU let the dot products of
// the rows that have arrived overlap the loads still in flight.
template <int SCHEME, int NBJ, int RW>
__device__ __forceinline__ void down_t1_slots_body(const ExpertsDev& ex, int k, const int32_t* __restrict__ idx,
                                                   const float* __restrict__ gate,
                                                   const uint16_t* __restrict__ h16, float* __restrict__ y, int bid) {
  __shared__ float part[kMaxK][4 * RW];
  const int tid = (int)threadIdx.x;
  const int q = tid >> 6, lane = tid & 63, lg = lane >> 4, ll = lane & 15;
  const int H = ex.H, I = ex.I, NBI = I / 32;
  const int mb = (int)bid * 4 * RW, m0 = mb + lg * RW;
  MOE_STAMP(g_stamps_decode, 4, bid);
  const int64_t rb = row_bytes<SCHEME>(I);
  // idx holds weight indices, or expert ids mapped here through a slot table;
  // an expert without a slot contributes nothing. The index is requested
  // first, so that waiting for it does not wait for the h loads too.
  const int iq = idx[q];
  XBlockH<SCHEME> hb[NBJ];
#pragma unroll
  for (int j = 0; j < NBJ; ++j) hb[j] = load_xblock_h<SCHEME>(h16, (int64_t)q * I, min(ll + 16 * j, NBI - 1));
  int e = expert_index(ex, iq);
  const bool resident = e >= 0;  // a slot-less expert: zero scales, whatever slot 0 holds
  e = max(e, 0);
#ifdef MOE_STAMPS
  asm volatile("" ::"v"(e));  // the routing read is consumed before the stamp
#endif
  MOE_STAMP_LANDED(g_stamps_decode, 5, bid);
  Block<SCHEME> c[RW][NBJ];
  float sc[RW][NBJ];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int64_t row = (int64_t)e * H + min(m0 + r, H - 1);
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      const int b = min(ll + 16 * j, NBI - 1);
      c[r][j] = load_block<SCHEME>(ex.wd + row * rb, b);
      sc[r][j] = scale_or_zero(ex.sd + row * NBI + b, resident);
    }
  }
  MOE_STAMP_LANDED(g_stamps_decode, 6, bid);
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    float part_r = 0.0f;
#pragma unroll
    for (int j = 0; j < NBJ; ++j)
      part_r = fmaf(ll + 16 * j < NBI ? sc[r][j] : 0.0f, block_dot_h<SCHEME>(c[r][j], hb[j]), part_r);
    part_r = row_sum16(part_r);
    if (ll == 0) {
      if (gate) part[q][lg * RW + r] = part_r;
      else if (m0 + r < H) y[(int64_t)q * H + m0 + r] = part_r;
    }
  }
  if (!gate) return;
  __syncthreads();
  if (tid < 4 * RW && mb + tid < H) {
    float acc = 0.0f;
    for (int s = 0; s < k; ++s) acc = fmaf(gate[s], part[s][tid], acc);
    y[mb + tid] = acc;
  }
  MOE_STAMP(g_stamps_decode, 7, bid);
}

template <int SCHEME, int NBJ, int RW>
__global__ __launch_bounds__(1024) void k_down_t1_slots(ExpertsDev ex, int k, const int32_t* __restrict__ idx,
                                                       const float* __restrict__ gate,
                                                       const uint16_t* __restrict__ h16, float* __restrict__ y) {
  down_t1_slots_body<SCHEME, NBJ, RW>(ex, k, idx, gate, h16, y, blockIdx.x);
}

// General single-token down (any k, any I): KC slots' rows in flight at a
// time, h read from global memory.
template <int SCHEME, int NBJ>
__global__ __launch_bounds__(128) void k_down_t1(ExpertsDev ex, int k, const int32_t* __restrict__ idx,
                                                 const float* __restrict__ gate, const float* __restrict__ h,
                                                 float* __restrict__ y) {
  constexpr int KC = NBJ >= 8 ? 1 : 8 / NBJ;
  const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
  const int lg = lane >> 4, ll = lane & 15;
  const int H = ex.H, I = ex.I, NBI = I / 32;
  const int m = ((int)blockIdx.x * 2 + wave) * 4 + lg;
  const int mm = min(m, H - 1);
  const int64_t rb = row_bytes<SCHEME>(I);
  float acc = 0.0f;
  for (int s0 = 0; s0 < k; s0 += KC) {
    Block<SCHEME> c[KC][NBJ];
    float sc[KC][NBJ];
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      const int ei = expert_index(ex, idx[min(s0 + q, k - 1)]);  // -1: no slot, contributes nothing
      const int64_t row = (int64_t)max(ei, 0) * H + mm;
#pragma unroll
      for (int j = 0; j < NBJ; ++j) {
        const int b = min(ll + 16 * j, NBI - 1);
        c[q][j] = load_block<SCHEME>(ex.wd + row * rb, b);
        sc[q][j] = scale_or_zero(ex.sd + row * NBI + b, ei >= 0);
      }
    }
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      const int s = s0 + q;
      if (s < k) {
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
            part = fmaf(sc[q][j], block_dot<SCHEME>(c[q][j], hv), part);
          }
        }
        part = row_sum16(part);
        if (gate) acc = fmaf(gate[s], part, acc);
        else if (ll == 0 && m < H) y[(int64_t)s * H + m] = part;
      }
    }
  }
  if (gate && ll == 0 && m < H) y[m] = acc;
}

// ------------------------------------------------------------------ T > 1, grouped
// Rows staged in LDS: each 32-element block of a row is followed by 16 bytes of
// padding, so the lanes of a wave (each reading its own block) spread over the
// banks. Copies go in 16-byte chunks, 8 loads per thread issued before their
// stores.
__device__ __forceinline__ int lds_block_stride(int elem_bytes) { return 32 * elem_bytes + 16; }

template <typename SrcRow>
__device__ __forceinline__ void stage_rows(uint8_t* lds, int row_stride, int nrow, int elems, int elem_bytes,
                                           SrcRow src_row) {
  const int blk = 32 * elem_bytes, cpb = blk / 16, pblk = blk + 16;
  const int chunks = elems * elem_bytes / 16, total = nrow * chunks;
  const int tid = (int)threadIdx.x, nth = (int)blockDim.x;
  for (int base = 0; base < total; base += 8 * nth) {
    uint4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = min(base + q * nth + tid, total - 1);
      v[q] = *reinterpret_cast<const uint4*>(src_row(c / chunks) + 16 * (c % chunks));
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = base + q * nth + tid;
      if (c < total) {
        const int i = c / chunks, j = c % chunks;
        *reinterpret_cast<uint4*>(lds + i * row_stride + (j / cpb) * pblk + 16 * (j % cpb)) = v[q];
      }
    }
  }
}

// Activations of block b from an LDS row (layout of stage_rows).
template <int SCHEME, int XT>
__device__ __forceinline__ void xreg_from_lds(XReg<SCHEME, XT>& r, const uint8_t* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  if constexpr (XT == MOE_F16) {
    uint32_t nat[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = q[i];
      nat[4 * i] = v.x; nat[4 * i + 1] = v.y; nat[4 * i + 2] = v.z; nat[4 * i + 3] = v.w;
    }
    r.h = xblock_from_pairs<SCHEME>(nat);
  } else if constexpr (XT == MOE_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = q[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r.f[8 * i + 2 * j] = bf16_bits_to_f32((uint16_t)(w[j] & 0xFFFF));
        r.f[8 * i + 2 * j + 1] = bf16_bits_to_f32((uint16_t)(w[j] >> 16));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = reinterpret_cast<const float4*>(p)[i];
      r.f[4 * i] = v.x; r.f[4 * i + 1] = v.y; r.f[4 * i + 2] = v.z; r.f[4 * i + 3] = v.w;
    }
  }
}

// Grid: (blocks_per_u, max unique experts). Workgroup column u serves expert
// uniq[u] for all of its n_e assignments: the code rows are loaded once, the
// routed tokens' activations are staged in LDS CH at a time, and every row is
// dotted with each of them, so a batch reads each routed expert once.
template <int SCHEME, int XT, int NBJ, int RP>
__global__ __launch_bounds__(256) void k_gate_up_grouped(const void* __restrict__ x, ExpertsDev ex, int k,
                                                         const int32_t* __restrict__ uniq,
                                                         const int32_t* __restrict__ n_uniq,
                                                         const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ perm, float* __restrict__ h,
                                                         int CH) {
  extern __shared__ uint8_t xs[];
  const int u = blockIdx.y;
  if (u >= *n_uniq) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = uniq[u], cnt = counts[e], beg = offsets[e];
  const int ew = expert_index(ex, e);  // -1: no slot, contributes nothing
  const int H = ex.H, I = ex.I, NB = H / 32;
  const int n0 = (blockIdx.x * 4 + wave) * RP;
  const int64_t rb = row_bytes<SCHEME>(H);
  Block<SCHEME> cg[RP][NBJ], cu[RP][NBJ];
  float sg[RP][NBJ], su[RP][NBJ];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int n = min(n0 + r, I - 1);
    const int64_t grow = (int64_t)max(ew, 0) * 2 * I + n, urow = grow + I;
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      const int b = min(lane + 64 * j, NB - 1);
      const bool valid = lane + 64 * j < NB && ew >= 0;
      cg[r][j] = load_block<SCHEME>(ex.wgu + grow * rb, b);
      cu[r][j] = load_block<SCHEME>(ex.wgu + urow * rb, b);
      sg[r][j] = scale_or_zero(ex.sgu + grow * NB + b, valid);
      su[r][j] = scale_or_zero(ex.sgu + urow * NB + b, valid);
    }
  }
  constexpr int xbytes = XT == MOE_F32 ? 4 : 2;
  const int pblk = lds_block_stride(xbytes), stride = NB * pblk;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  for (int a0 = 0; a0 < cnt; a0 += CH) {
    const int nt = min(CH, cnt - a0);
    __syncthreads();
    stage_rows(xs, stride, nt, H, xbytes,
               [&](int i) { return xb + (int64_t)(perm[beg + a0 + i] / k) * H * xbytes; });
    __syncthreads();
    for (int i = 0; i < nt; ++i) {
      const int f = perm[beg + a0 + i];
      float ag[RP], au[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) ag[r] = au[r] = 0.0f;
#pragma unroll
      for (int j = 0; j < NBJ; ++j) {
        XReg<SCHEME, XT> xr;
        xreg_from_lds<SCHEME, XT>(xr, xs + i * stride + min(lane + 64 * j, NB - 1) * pblk);
#pragma unroll
        for (int r = 0; r < RP; ++r) {
          ag[r] = fmaf(sg[r][j], xdot<SCHEME, XT>(cg[r][j], xr), ag[r]);
          au[r] = fmaf(su[r][j], xdot<SCHEME, XT>(cu[r][j], xr), au[r]);
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
}

// Grid: (ceil(H / 16), max unique experts). ys[f][m] = row m of expert uniq[u] . h[f]
// for each assignment f of that expert; the h rows are staged in LDS CH at a time.
template <int SCHEME, int NBJ>
__global__ __launch_bounds__(256) void k_down_grouped(ExpertsDev ex, int k, const int32_t* __restrict__ uniq,
                                                      const int32_t* __restrict__ n_uniq,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ perm, const float* __restrict__ h,
                                                      float* __restrict__ ys, int CH) {
  extern __shared__ uint8_t hsm[];
  const int u = blockIdx.y;
  if (u >= *n_uniq) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lg = lane >> 4, ll = lane & 15;
  const int e = uniq[u], cnt = counts[e], beg = offsets[e];
  const int ew = expert_index(ex, e);  // -1: no slot, contributes nothing
  const int H = ex.H, I = ex.I, NBI = I / 32;
  const int m = (blockIdx.x * 4 + wave) * 4 + lg;
  const int mm = min(m, H - 1);
  const int64_t rb = row_bytes<SCHEME>(I);
  const int64_t row = (int64_t)max(ew, 0) * H + mm;
  Block<SCHEME> c[NBJ];
  float sc[NBJ];
#pragma unroll
  for (int j = 0; j < NBJ; ++j) {
    const int b = min(ll + 16 * j, NBI - 1);
    c[j] = load_block<SCHEME>(ex.wd + row * rb, b);
    sc[j] = scale_or_zero(ex.sd + row * NBI + b, ll + 16 * j < NBI && ew >= 0);
  }
  const int pblk = lds_block_stride(4), stride = NBI * pblk;
  const uint8_t* hb = reinterpret_cast<const uint8_t*>(h);
  for (int a0 = 0; a0 < cnt; a0 += CH) {
    const int nt = min(CH, cnt - a0);
    __syncthreads();
    stage_rows(hsm, stride, nt, I, 4, [&](int i) { return hb + (int64_t)perm[beg + a0 + i] * I * 4; });
    __syncthreads();
    for (int i = 0; i < nt; ++i) {
      const int f = perm[beg + a0 + i];
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < NBJ; ++j) {
        const int b = min(ll + 16 * j, NBI - 1);
        float hv[32];
        const float4* hp = reinterpret_cast<const float4*>(hsm + i * stride + b * pblk);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float4 v = hp[q];
          hv[4 * q] = v.x; hv[4 * q + 1] = v.y; hv[4 * q + 2] = v.z; hv[4 * q + 3] = v.w;
        }
        part = fmaf(sc[j], block_dot<SCHEME>(c[j], hv), part);
      }
      part = row_sum16(part);
      if (ll == 0 && m < H) ys[(int64_t)f * H + m] = part;
    }
  }
}

// y[t][m] = sum over slots s, in order, of gate[t][s] * ys[t*k+s][m], with the
// per-slot rows in fp32 (ys) or, with HALF, as the grouped GEMM stores them:
// fp16 (ys16) times 2^ysig[t*k+s][m/32], exact powers of two. Four
// consecutive outputs of one token per thread; every slot's loads are issued
// before the fused multiply-adds, which run in slot order (KMAX >= k). With NT
// the fp32 rows are read non-temporally (rows larger than the cache that would
// hold them).
template <int KMAX, bool HALF, bool NT>
__global__ __launch_bounds__(256) void k_combine(int T, int H, int k, const float* __restrict__ gate,
                                                 const float* __restrict__ ys, const uint16_t* __restrict__ ys16,
                                                 const int32_t* __restrict__ ysig, float* __restrict__ y) {
  const int nbx = (H / 4 + 255) / 256;
  const int t = blockIdx.x / nbx;
  const int m = ((blockIdx.x % nbx) * 256 + threadIdx.x) * 4;
  if (t >= T || m >= H) return;
  float4 v[KMAX];
  float g[KMAX];
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    const int sc = min(s, k - 1);
    const int64_t off = ((int64_t)t * k + sc) * H + m;
    if constexpr (HALF) {
      const uint2 u = *reinterpret_cast<const uint2*>(ys16 + off);
      const int e = ysig[((int64_t)t * k + sc) * (H / 32) + m / 32];
      const half2v lo = as_h2(u.x), hi = as_h2(u.y);
      v[s] = make_float4(ldexpf((float)lo[0], e), ldexpf((float)lo[1], e), ldexpf((float)hi[0], e),
                         ldexpf((float)hi[1], e));
    } else if constexpr (NT) {
      typedef float f4v __attribute__((ext_vector_type(4)));
      const f4v q = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(ys + off));
      v[s] = make_float4(q[0], q[1], q[2], q[3]);
    } else {
      v[s] = *reinterpret_cast<const float4*>(ys + off);
    }
    g[s] = gate[(int64_t)t * k + sc];
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    if (s < k) {
      acc.x = fmaf(g[s], v[s].x, acc.x);
      acc.y = fmaf(g[s], v[s].y, acc.y);
      acc.z = fmaf(g[s], v[s].z, acc.z);
      acc.w = fmaf(g[s], v[s].w, acc.w);
    }
  }
  *reinterpret_cast<float4*>(y + (int64_t)t * H + m) = acc;
}

// ------------------------------------------------------------------ launchers
// The single-token down kernel: one wave per slot (fp16 h) for I <= 1024, the
// general kernel (fp32 h) above that.
constexpr int kDownRows = 2;

hipError_t launch_decode_t1(const void* x, int xtype, const ExpertsDev& ex, int k, int renorm,
                            const float* logits, const int32_t* idx_in, const float* gate_in,
                            int32_t* idx_ws, float* gate_ws, int32_t* idx_user, float* gate_user,
                            float* h, float* y, bool h32, hipStream_t s) {
  const bool from_logits = logits != nullptr;
  const int nbi = (ex.I / 32 + 15) / 16;
  // fp16 h and the one-wave-per-slot down kernel, unless fp32 h is asked for
  const bool slots = nbi <= 2 && !h32;
  const int nbj = (ex.H / 32 + 63) / 64;  // 1 (H <= 2048) or 2 (H <= 4096)
  with_scheme(ex.scheme, [&](auto S) {
    with_xtype(xtype, [&](auto X) {
      constexpr int SC = decltype(S)::value, XT = decltype(X)::value;
      auto go = [&](auto NBJc, auto RPc) {
        constexpr int NBJ = decltype(NBJc)::value, RP = decltype(RPc)::value;
        const int bps = (ex.I + kGateUpWaves * RP - 1) / (kGateUpWaves * RP);
        // from logits: one more workgroup, which publishes the routing
        dim3 grid(k * bps + (from_logits ? 1 : 0));
        auto launch = [&](auto RTc, auto VPLc, auto H16c) {
          constexpr bool H16 = decltype(H16c)::value != 0;
          constexpr int RT = decltype(RTc)::value, VPL = decltype(VPLc)::value;
          MOE_LAUNCH(MOE_KERNEL_GATE_UP, (k_gate_up_t1<SC, XT, NBJ, RP, RT, VPL, H16>), grid, dim3(64 * kGateUpWaves), 0, s, x, ex,
                     k, renorm, logits, idx_in, idx_ws, gate_ws, idx_user, gate_user, h, bps);
        };
        auto with_h = [&](auto RTc, auto VPLc) {
          if (slots) launch(RTc, VPLc, IC<1>{});
          else launch(RTc, VPLc, IC<0>{});
        };
        // the top-k over a slot table is a kernel of its own, so that the
        // plain one carries none of its code
        auto with_vpl = [&](auto RTc) {
          if (ex.E <= 256) with_h(RTc, IC<4>{});
          else if (ex.E <= 512) with_h(RTc, IC<8>{});
          else with_h(RTc, IC<16>{});
        };
        if (!from_logits) with_h(IC<0>{}, IC<1>{});
        else if (ex.slot_of) with_vpl(IC<2>{});
        else with_vpl(IC<1>{});
      };
      if (nbj <= 1) go(IC<1>{}, IC<1>{});
      else go(IC<2>{}, IC<1>{});
    });
  });
  const int32_t* idx = from_logits ? idx_ws : idx_in;
  const float* gate = from_logits ? gate_ws : gate_in;
  // from logits, gate/up publishes weight indices (slots when staged): the
  // down kernel takes them as they are
  ExpertsDev exd = ex;
  if (from_logits) exd.slot_of = nullptr;
  with_scheme(ex.scheme, [&](auto S) {
    constexpr int SC = decltype(S)::value;
    if (slots) {
      dim3 grid((ex.H + 4 * kDownRows - 1) / (4 * kDownRows));
      const uint16_t* h16 = reinterpret_cast<const uint16_t*>(h);
      if (nbi <= 1)
        MOE_LAUNCH(MOE_KERNEL_DOWN, (k_down_t1_slots<SC, 1, kDownRows>), grid, dim3(64 * k), 0, s, exd, k, idx, gate,
                   h16, y);
      else
        MOE_LAUNCH(MOE_KERNEL_DOWN, (k_down_t1_slots<SC, 2, kDownRows>), grid, dim3(64 * k), 0, s, exd, k, idx, gate,
                   h16, y);
      return;
    }
    dim3 grid((ex.H + 7) / 8);
    auto go = [&](auto NBJc) {
      constexpr int NBJ = decltype(NBJc)::value;
      MOE_LAUNCH(MOE_KERNEL_DOWN, (k_down_t1<SC, NBJ>), grid, dim3(128), 0, s, exd, k, idx, gate, h, y);
    };
    if (nbi <= 4) go(IC<4>{});
    else go(IC<8>{});
  });
  return hipGetLastError();
}

// ------------------------------------------------------------------ prerouted decode, T = 1
// Prediction as routing ("The Other Half of the Memory Wall: Serving 35B MoEs
// from SSD with Trained Routing Prediction", xyznot.com, section 主なアイデア):
// a layer runs its experts on the logits its predecessor's head predicted, and
// its own head predicts the next layer's. The head's stage 1 needs only the
// layer input and the layer's routing, and its stage 2 only stage 1's output,
// so each joins an expert launch as extra workgroups ahead of the expert grid.
// Two launches per layer, against the router path's three.

// F + E head rows (fc1 + GELU, residual path), then the gate/up grid; the head
// rows come first so their weight reads, which do not wait for the routing,
// start with the launch. A head workgroup picks the layer's routing from the
// same logits, as the gate/up workgroups do, for the current-token k-hot
// input, while those reads are in flight.
template <int SCHEME, int XT, int NBJ, int VPL, int HNCH>
__global__ __launch_bounds__(64 * kGateUpWaves) void k_gate_up_t1_head(
    const void* __restrict__ x, ExpertsDev ex, int k, int renorm, const float* __restrict__ logits,
    int32_t* __restrict__ idx_ws, float* __restrict__ gate_ws, int32_t* __restrict__ idx_user,
    float* __restrict__ gate_user, float* __restrict__ h, int blocks_per_slot, HeadDev hd,
    const int32_t* __restrict__ prev, float* __restrict__ act, float* __restrict__ part) {
  static_assert(kGateUpWaves == kHeadWaves, "head rows run on gate/up-sized workgroups");
  const int nhead = hd.F + hd.E;
  if ((int)blockIdx.x >= nhead) {
    gate_up_t1_body<SCHEME, XT, NBJ, 1, 1, VPL, true>(x, ex, k, renorm, logits, nullptr, idx_ws, gate_ws, idx_user,
                                                         gate_user, h, blocks_per_slot, (int)blockIdx.x - nhead);
    return;
  }
  head_stage1_t1_routed<XT, HNCH, VPL>((int)blockIdx.x, x, hd.H, hd.E, hd.F, hd.w1, hd.b1, hd.wl, hd.b2, logits, k,
                                       renorm, prev, act, part);
}

// ceil(E / k) workgroups of head stage 2 (one fc2 row per wave), then the down
// grid.
template <int SCHEME, int NBJ, int RW, int HNCHF>
__global__ __launch_bounds__(1024) void k_down_t1_slots_head(ExpertsDev ex, int k, const int32_t* __restrict__ idx,
                                                            const float* __restrict__ gate,
                                                            const uint16_t* __restrict__ h16, float* __restrict__ y,
                                                            int nmain, const float* __restrict__ act,
                                                            const float* __restrict__ part,
                                                            const float* __restrict__ w2, int E, int F,
                                                            float* __restrict__ logits_next) {
  const int nhead = (int)gridDim.x - nmain;
  if ((int)blockIdx.x >= nhead) {
    down_t1_slots_body<SCHEME, NBJ, RW>(ex, k, idx, gate, h16, y, (int)blockIdx.x - nhead);
    return;
  }
  head_stage2_body<HNCHF, 1>((int)blockIdx.x, 0, (int)(blockDim.x >> 6), act, part, w2, 1, E, F, logits_next);
}

bool prerouted_t1_fusable(const ExpertsDev& ex, int xtype, const HeadDev& hd) {
  const int nbi = (ex.I / 32 + 15) / 16;
  return nbi <= 2 && hd.E == ex.E && hd.H == ex.H && hd.F <= 1024 && (xtype == MOE_F16 || xtype == MOE_BF16 ||
                                                                       xtype == MOE_F32);
}

hipError_t launch_prerouted_t1(const void* x, int xtype, const ExpertsDev& ex, int k, int renorm,
                               const float* logits, int32_t* idx_ws, float* gate_ws, int32_t* idx_user,
                               float* gate_user, float* h, float* y, const HeadDev& hd, const int32_t* prev,
                               float* act, float* part, float* logits_next, hipStream_t s) {
  const int nbi = (ex.I / 32 + 15) / 16;
  const int nbj = (ex.H / 32 + 63) / 64;
  const int hnch = ((hd.H + 255) / 256 + kHeadWaves - 1) / kHeadWaves;
  with_scheme(ex.scheme, [&](auto S) {
    with_xtype(xtype, [&](auto X) {
      constexpr int SC = decltype(S)::value, XT = decltype(X)::value;
      auto go = [&](auto NBJc, auto VPLc, auto HNc) {
        constexpr int NBJ = decltype(NBJc)::value, VPL = decltype(VPLc)::value, HN = decltype(HNc)::value;
        const int bps = (ex.I + kGateUpWaves - 1) / kGateUpWaves;
        dim3 grid(k * bps + 1 + hd.F + hd.E);  // the expert grid ends with its routing publisher
        MOE_LAUNCH(MOE_KERNEL_GATE_UP, (k_gate_up_t1_head<SC, XT, NBJ, VPL, HN>), grid, dim3(64 * kGateUpWaves), 0, s,
                   x, ex, k, renorm, logits, idx_ws, gate_ws, idx_user, gate_user, h, bps, hd, prev, act, part);
      };
      auto with_hn = [&](auto NBJc, auto VPLc) {
        if (hnch <= 1) go(NBJc, VPLc, IC<1>{});
        else if (hnch <= 2) go(NBJc, VPLc, IC<2>{});
        else go(NBJc, VPLc, IC<4>{});
      };
      auto with_v = [&](auto NBJc) {
        if (ex.E <= 256) with_hn(NBJc, IC<4>{});
        else if (ex.E <= 512) with_hn(NBJc, IC<8>{});
        else with_hn(NBJc, IC<16>{});
      };
      if (nbj <= 1) with_v(IC<1>{});
      else with_v(IC<2>{});
    });
  });
  const int hnchf = (hd.F + 255) / 256;
  with_scheme(ex.scheme, [&](auto S) {
    constexpr int SC = decltype(S)::value;
    const int nmain = (ex.H + 4 * kDownRows - 1) / (4 * kDownRows);
    dim3 grid(nmain + (hd.E + k - 1) / k);
    const uint16_t* h16 = reinterpret_cast<const uint16_t*>(h);
    auto go = [&](auto NBIc, auto HFc) {
      constexpr int NBI = decltype(NBIc)::value, HF = decltype(HFc)::value;
      MOE_LAUNCH(MOE_KERNEL_DOWN, (k_down_t1_slots_head<SC, NBI, kDownRows, HF>), grid, dim3(64 * k), 0, s, ex, k,
                 idx_ws, gate_ws, h16, y, nmain, act, part, hd.w2, hd.E, hd.F, logits_next);
    };
    auto with_hf = [&](auto NBIc) {
      if (hnchf <= 1) go(NBIc, IC<1>{});
      else if (hnchf <= 2) go(NBIc, IC<2>{});
      else go(NBIc, IC<4>{});
    };
    if (nbi <= 1) with_hf(IC<1>{});
    else with_hf(IC<2>{});
  });
  return hipGetLastError();
}

// Rows per LDS chunk for the grouped kernels: up to 16, within 64 KiB.
static int lds_chunk_rows(int row_stride) { return std::max(1, std::min(16, 65536 / row_stride)); }

hipError_t launch_decode_grouped(const void* x, int xtype, int T, const ExpertsDev& ex, int k,
                                 const GroupBufs& g, const float* gate, float* h, float* ys, float* y,
                                 hipStream_t s) {
  const int maxu = (int)std::min<int64_t>((int64_t)ex.E, (int64_t)T * k);
  const int nbj = (ex.H / 32 + 63) / 64;
  const int xbytes = xtype == MOE_F32 ? 4 : 2;
  const int xstride = ex.H / 32 * (32 * xbytes + 16);
  const int xch = lds_chunk_rows(xstride);
  with_scheme(ex.scheme, [&](auto S) {
    with_xtype(xtype, [&](auto X) {
      constexpr int SC = decltype(S)::value, XT = decltype(X)::value;
      auto go = [&](auto NBJc, auto RPc) {
        constexpr int NBJ = decltype(NBJc)::value, RP = decltype(RPc)::value;
        dim3 grid((ex.I + 4 * RP - 1) / (4 * RP), maxu);
        MOE_LAUNCH(MOE_KERNEL_GATE_UP, (k_gate_up_grouped<SC, XT, NBJ, RP>), grid, dim3(256),
                   (size_t)xch * xstride, s, x, ex, k, g.uniq, g.n_uniq, g.counts, g.offsets, g.perm, h, xch);
      };
      if (nbj <= 1) go(IC<1>{}, IC<4>{});
      else go(IC<2>{}, IC<2>{});
    });
  });
  float* out = gate ? ys : y;  // per-slot mode writes [T][k][H] directly
  const int nbi = (ex.I / 32 + 15) / 16;
  const int hstride = ex.I / 32 * (32 * 4 + 16);
  const int hch = lds_chunk_rows(hstride);
  const size_t hlds = (size_t)hch * hstride;
  dim3 grid((ex.H + 15) / 16, maxu);
  with_scheme(ex.scheme, [&](auto S) {
    constexpr int SC = decltype(S)::value;
    auto go = [&](auto NBJc) {
      constexpr int NBJ = decltype(NBJc)::value;
      MOE_LAUNCH(MOE_KERNEL_DOWN, (k_down_grouped<SC, NBJ>), grid, dim3(256), hlds, s, ex, k, g.uniq, g.n_uniq,
                 g.counts, g.offsets, g.perm, h, out, hch);
    };
    if (nbi <= 1) go(IC<1>{});
    else if (nbi <= 2) go(IC<2>{});
    else if (nbi <= 4) go(IC<4>{});
    else go(IC<8>{});
  });
  if (gate) return launch_combine(T, ex.H, k, gate, ys, nullptr, nullptr, y, s);
  return hipGetLastError();
}

hipError_t launch_combine(int T, int H, int k, const float* gate, const float* ys, const uint16_t* ys16,
                          const int32_t* ysig, float* y, hipStream_t s) {
  const dim3 cg((unsigned)((int64_t)T * ((H / 4 + 255) / 256)));
  auto go = [&](auto KM, auto HF, auto NTc) {
    constexpr int K_ = decltype(KM)::value;
    constexpr bool H_ = decltype(HF)::value != 0, N_ = decltype(NTc)::value != 0;
    MOE_LAUNCH(MOE_KERNEL_COMBINE, (k_combine<K_, H_, N_>), cg, dim3(256), 0, s, T, H, k, gate, ys, ys16, ysig, y);
  };
  // Per-slot rows beyond the 256 MB last-level cache are read non-temporally:
  // measured faster there (8192 tokens, 537 MB) and slower below (2048, 134 MB).
  const bool nt = (int64_t)T * k * H * 4 > ((int64_t)256 << 20);
  if (ys16) {
    if (k <= 8) go(IC<8>{}, IC<1>{}, IC<0>{});
    else go(IC<16>{}, IC<1>{}, IC<0>{});
  } else if (nt) {
    if (k <= 8) go(IC<8>{}, IC<0>{}, IC<1>{});
    else go(IC<16>{}, IC<0>{}, IC<1>{});
  } else {
    if (k <= 8) go(IC<8>{}, IC<0>{}, IC<0>{});
    else go(IC<16>{}, IC<0>{}, IC<0>{});
  }
  return hipGetLastError();
}

}  // namespace moe

MOE_STAMP_READER(moe_stamps_read_decode, moe::g_stamps_decode);
