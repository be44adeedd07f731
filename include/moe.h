/*
 * moe.h — C ABI of the MI355X (gfx950) routed, block-quantized MoE expert layer.
 *
 * The layer, as the pages describe it:
 *   [LR] "QwenのMoEルーターを観測してホットエキスパートを先読みしても速くならなかった"
 *        (lilting.ch). Section "ルーターをフックする" (hooking the router): the router
 *        is a gate linear, a precise softmax and a top-k. Section
 *        "事前ウォームアップとmmapキャッシュを比べる": expert weights are one stacked
 *        (experts, output_dims, input_dims) array, and gather_qmm multiplies by
 *        the experts named in rhs_indices.
 *   [QK] "鳴かぬなら、カスタムカーネル、ほととぎす" (qiita.com, john-rocky).
 *        Section 1: an MoE token runs only its top-k experts, so decode should
 *        read only those experts' weights. Section 4: the routed expert ids are
 *        a kernel input and index the weight reads, so unrouted experts are never
 *        fetched. Section 6: weights are symmetric linear int8 with one scale per
 *        32 K elements ("sym8"). Section 7: gate and up share the token, while
 *        the down projection of each slot takes that expert's own gated
 *        activation.
 *
 * Conventions, common to every entry point:
 *   - Array arguments are DEVICE pointers to memory the caller owns. The library
 *     keeps no pointer after a call returns. The moe_experts struct itself is
 *     read on the host, during the call only.
 *   - Every call is asynchronous on `stream`, a hipStream_t passed as void*
 *     (NULL means the default stream). No call allocates device memory or
 *     copies device data to the host, and none synchronises except the
 *     benchmark timer's moe_timer_read.
 *   - Arguments are checked on the host before any launch. A failed check
 *     returns an error and launches nothing. moe_last_error() then describes it,
 *     per calling thread.
 *   - Scratch memory comes from the caller: `ws` must hold at least
 *     moe_workspace_bytes(...) bytes, aligned to 256 bytes. Calls that share a
 *     workspace must be ordered, for example on one stream.
 *   - Layouts are row-major and C-contiguous. Device arrays must be 16-byte
 *     aligned.
 *   - Codes: sym8 stores one int8 two's-complement code per byte, in K order.
 *     int4 stores two codes per byte: the even K index in the low nibble, the
 *     odd one in the high nibble, each a two's-complement nibble in [-7, 7].
 *     Scales are IEEE binary16 bit patterns, one per 32 consecutive K elements
 *     of a row. A weight is code * scale.
 *   - Limits: 1 <= T <= 65536; 32 <= H <= 4096 and 32 <= I <= 4096, both
 *     multiples of 32; 1 <= E <= 1024; 1 <= k <= min(E, 16).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, a shape outside the limits, misalignment */
  MOE_ERR_UNSUPPORTED = 2,  /* unknown dtype, codec or flag */
  MOE_ERR_WORKSPACE = 3,    /* ws too small, or not 256-byte aligned */
  MOE_ERR_HIP = 4           /* a HIP launch failed; moe_last_error() names it */
} moe_status;

/* Activation element type of x. */
typedef enum { MOE_F32 = 0, MOE_F16 = 1, MOE_BF16 = 2 } moe_dtype;

/* Weight codec [QK §6, §3/§7]: sym8 codes lie in [-127, 127], int4 codes in [-7, 7]. */
typedef enum { MOE_Q_SYM8 = 0, MOE_Q_INT4 = 1 } moe_qscheme;

enum {
  /* Renormalise the k gates of each token so they sum to one. */
  MOE_FLAG_RENORM = 1u,
  /* Expert-path selection; with neither bit set the library uses the gathered
   * matvec kernels for T == 1 and for fp32 activations, and the grouped MFMA
   * GEMM for T > 1 with fp16 or bf16 activations.
   * GATHER: gathered matvec kernels (exact code * scale products, fp32 sums).
   * GEMM: grouped MFMA GEMM on the raw codes, one 32-element block per MFMA
   *       step, each block's fp32 partial times its scale (weights exact); the
   *       activations are the other operand as given (fp16 or bf16; fp32 x is
   *       MOE_ERR_UNSUPPORTED with this bit); h is held in fp16 with a
   *       power-of-two exponent per tile, so no intermediate overflows; the
   *       per-slot outputs ahead of the combine are fp32, or, where those fp32
   *       rows (T*k*H*4 bytes) would exceed 256 MB, fp16 with a power-of-two
   *       exponent per row and 32 columns (the per-slot output returned with
   *       topk_gate == NULL is always fp32). */
  MOE_FLAG_PATH_GATHER = 2u,
  MOE_FLAG_PATH_GEMM = 4u,
  /* Single-token path only: keep h = silu(gate) * up in fp32 between the
   * gate/up and down kernels (by default it is stored in fp16, rounded to
   * nearest even, when I <= 1024, and the down kernel reads half the bytes).
   * Ignored by the T > 1 paths; moe_prerouted_layer_forward with this bit runs
   * its expert and head launches separately (the fused form holds h in fp16). */
  MOE_FLAG_H_FP32 = 8u
};

/* Stacked experts [LR "事前ウォームアップとmmapキャッシュを比べる"]:
 *   w_gate_up: [E][2I][H] codes (int4: [E][2I][H/2] bytes). Rows 0..I-1 of an
 *              expert are the gate projection and rows I..2I-1 the up projection.
 *   s_gate_up: [E][2I][H/32] binary16 scales.
 *   w_down:    [E][H][I] codes (int4: [E][H][I/2] bytes).
 *   s_down:    [E][H][I/32] binary16 scales.                                  */
typedef struct moe_experts {
  int32_t E, H, I;
  int32_t scheme;           /* moe_qscheme */
  const void* w_gate_up;
  const uint16_t* s_gate_up;
  const void* w_down;
  const uint16_t* s_down;
} moe_experts;

/* Bytes of workspace that moe_route, moe_gather_qmm_forward and
 * moe_layer_forward need for these sizes, with any flags. Returns 0 when the
 * sizes are outside the limits. */
size_t moe_workspace_bytes(int32_t T, int32_t E, int32_t H, int32_t I, int32_t k, int32_t scheme);

/* Router [LR "ルーターをフックする"]: logits = x R^T in fp32, a softmax over the E
 * experts and the top k.
 *   x:         [T][H] activations of type xtype.
 *   router_w:  [E][H] fp32.
 *   topk_idx:  out [T][k] int32. Expert ids by descending logit, ties to the
 *              lower id.
 *   topk_gate: out [T][k] fp32. Softmax probability of each chosen expert,
 *              divided by their sum when flags has MOE_FLAG_RENORM. */
moe_status moe_route(const void* x, int32_t xtype, int32_t T, int32_t H, const float* router_w,
                     int32_t E, int32_t k, uint32_t flags, int32_t* topk_idx, float* topk_gate,
                     void* ws, size_t ws_bytes, void* stream);

/* Token-by-expert grouping of the T*k assignments f = t*k + s of topk_idx.
 * This is the step that lets a batch read each routed expert once.
 *   counts:  out [E]     assignments per expert.
 *   offsets: out [E+1]   exclusive prefix sum of counts.
 *   perm:    out [T*k]   flat ids ordered by expert, then by f.
 *   uniq:    out [E]     experts with counts > 0, ascending. Entries past
 *                        *n_uniq are unspecified.
 *   n_uniq:  out [1]     number of such experts.
 * topk_idx entries must lie in [0, E) and the k ids of one token must be
 * distinct, as moe_route produces them; the caller guarantees both. `ws` must
 * hold moe_workspace_bytes(T, E, 32, 32, k, 0) bytes. */
moe_status moe_group(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* uniq, int32_t* n_uniq,
                     void* ws, size_t ws_bytes, void* stream);

/* Gathered quantized expert layer, the routed-only gather_qmm [QK §4, §7;
 * LR "事前ウォームアップとmmapキャッシュを比べる"]. For each token t and slot s,
 * with e = topk_idx[t][s]:
 *   u = W_gu[e] x_t (2I values); h = silu(u[0:I]) * u[I:2I], where
 *   silu(z) = z / (1 + exp(-z)); ys = W_d[e] h.
 * Only the weights of experts named in topk_idx are read.
 *   topk_gate: [T][k] fp32. With it, y is [T][H] = sum_s gate[t][s] * ys, in
 *              slot order. With topk_gate == NULL, y is [T][k][H], the per-slot ys.
 *   topk_idx:  entries must lie in [0, E), and the k ids of one token must be
 *              distinct, as moe_route produces them. The caller guarantees
 *              both; they are not checked on the device.
 *   flags:     MOE_FLAG_PATH_* bits select the path; other bits are ignored. */
moe_status moe_gather_qmm_forward(const void* x, int32_t xtype, int32_t T, const moe_experts* ex,
                                  int32_t k, const int32_t* topk_idx, const float* topk_gate,
                                  float* y, uint32_t flags, void* ws, size_t ws_bytes, void* stream);

/* Whole expert layer: moe_route, then moe_gather_qmm_forward on its output.
 *   y:             out [T][H] fp32.
 *   topk_idx_out:  out [T][k], or NULL.
 *   topk_gate_out: out [T][k], or NULL.                                        */
moe_status moe_layer_forward(const void* x, int32_t xtype, int32_t T, const float* router_w,
                             const moe_experts* ex, int32_t k, uint32_t flags, float* y,
                             int32_t* topk_idx_out, float* topk_gate_out,
                             void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * scratch comes from a static device array of MOE_NOALLOC_SCRATCH_BYTES inside
 * the library instead of a caller workspace; every GPU the library runs on holds
 * its own copy until the process ends. The call itself allocates nothing: its
 * first call on a device, with that device current, looks the array's address
 * up once (hipGetSymbolAddress).
 *   Arguments, results and kernels are moe_layer_forward's. `stream` must belong
 *   to the current device (NULL: its default stream).
 *   Every call on one GPU shares that GPU's array and it keeps the last call's
 *   contents; nothing in it needs to start at zero. Calls that overlap on one
 *   GPU (two streams, two threads) race on it: order them, e.g. on one stream.
 * Errors: as moe_layer_forward's, and MOE_ERR_WORKSPACE when the sizes need more
 * than MOE_NOALLOC_SCRATCH_BYTES (moe_workspace_bytes(T, E, H, I, k, scheme)
 * must not exceed it: any single-token shape, and batches such as T = 64, E =
 * 512, H = 2048, I = 512, k = 10 fit), MOE_ERR_INVALID_ARG when `stream` is on
 * another device, MOE_ERR_HIP when the address lookup fails. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
moe_status moe_layer_forward_noalloc(const void* x, int32_t xtype, int32_t T, const float* router_w,
                                     const moe_experts* ex, int32_t k, uint32_t flags, float* y,
                                     int32_t* topk_idx_out, float* topk_gate_out, void* stream);

/* The expert layer from given router logits: moe_layer_forward after its gate
 * linear, for logits that come from elsewhere, such as moe_prerouter_forward
 * predicting this layer's routing (prediction as routing: "The Other Half of the
 * Memory Wall: Serving 35B MoEs from SSD with Trained Routing Prediction"
 * (xyznot.com), section 主なアイデア). The softmax and top-k run on `logits`
 * ([T][E] fp32, DEVICE, 16-byte aligned) exactly as moe_route's, then the routed
 * experts as moe_gather_qmm_forward's. For one token the top-k runs inside the
 * gate/up kernel. Other arguments and errors as moe_layer_forward's. */
moe_status moe_experts_from_logits(const void* x, int32_t xtype, int32_t T, const float* logits,
                                   const moe_experts* ex, int32_t k, uint32_t flags, float* y,
                                   int32_t* topk_idx_out, float* topk_gate_out,
                                   void* ws, size_t ws_bytes, void* stream);

/* Block quantiser for the codecs above [QK §6]: w [rows][K] fp32 to codes and
 * scales. Per block of 32: s = binary16(amax / qmax), with the division in
 * fp32, rounded to nearest even and saturated at the largest finite value;
 * then q = clamp(rint(w / s), -qmax, qmax) in fp32, or q = 0 when s == 0.
 *   codes:  out [rows][K] (sym8) or [rows][K/2] (int4) bytes.
 *   scales: out [rows][K/32] binary16.
 * K must be a positive multiple of 32. Non-finite inputs give unspecified codes. */
moe_status moe_quantize(const float* w, int64_t rows, int32_t K, int32_t scheme, void* codes,
                        uint16_t* scales, void* stream);

/* Benchmark support: per-launch kernel durations from HIP events.
 * moe_timer_start arms a timer for the next `capacity` launches of one kernel
 * family (MOE_KERNEL_*), on any stream; those launches go through
 * hipExtLaunchKernel with a start and a stop event. moe_timer_read waits for
 * the recorded launches (a host synchronisation, the only one in this
 * library), writes up to `capacity` durations in milliseconds to the host
 * array `ms`, stores how many were recorded in *count and disarms the timer.
 * Global state: not thread-safe, and not for launches under graph capture.
 * capacity must lie in [1, 1 << 20]. */
enum {
  MOE_KERNEL_ROUTE_LOGITS = 0,  /* router logits (GEMV or tiled GEMM) */
  MOE_KERNEL_TOPK = 1,          /* one-wave top-k */
  MOE_KERNEL_GROUP = 2,         /* token-by-expert grouping (three kernels) */
  MOE_KERNEL_GATE_UP = 3,       /* gathered gate/up + SwiGLU (one token or grouped) */
  MOE_KERNEL_DOWN = 4,          /* gathered per-slot down (+ combine for one token) */
  MOE_KERNEL_COMBINE = 5,       /* gate-weighted combine (T > 1) */
  MOE_KERNEL_GEMM_GATE_UP = 6,  /* grouped MFMA GEMM, gate/up + SwiGLU */
  MOE_KERNEL_GEMM_DOWN = 7,     /* grouped MFMA GEMM, down */
  MOE_KERNEL_QUANTIZE = 8,      /* block quantiser */
  MOE_KERNEL_HEAD = 9,          /* prerouter head rows (fc1 + GELU; fc2 + residual path) */
  MOE_KERNEL_LORA = 10,         /* quantized linear with LoRA delta (A x; W_q x + delta) */
  MOE_KERNEL_COUNT = 11
};
moe_status moe_timer_start(int32_t kernel, int32_t capacity);
moe_status moe_timer_read(float* ms, int32_t capacity, int32_t* count);

/* Expert-cache miss policies, replayed over a sequence of routings (host code).
 * "Which Expert Misses Are Worth Waiting For? Substitution and Caching for
 * Mixture-of-Experts Inference on a Consumer GPU" (gist.science), section 手法
 * (method): a routed expert that is not resident is fetched synchronously or
 * substituted by a resident one; MOE_MISS_FETCH_ALL fetches every miss,
 * MOE_MISS_RULE fetches a miss that is the first choice (slot 0) or has gate >=
 * `threshold` (0.15 on the page), MOE_MISS_FIRST_CHOICE fetches first-choice misses
 * only. With admit_beta > 0 each substituted expert's gates accumulate and it is
 * admitted in the background once the sum reaches admit_beta (0.5 on the page,
 * section 主な貢献と知見, item 5, with frequency-based eviction).
 * Cache: `capacity` slots (k <= capacity <= E), initially empty; an admission into
 * a full cache evicts the resident expert selected least often so far (lower id on
 * ties), never one the current token selected; an admission resets the expert's
 * accumulator.
 * Inputs: HOST arrays topk_idx [T][k] (slot order, ids in [0, E), distinct per
 * token) and topk_gate [T][k] (the normalised gates). Outputs, HOST arrays: m [T]
 * (substituted gate mass of each token), sync_fetches [T], bg_fetches [T] (experts
 * admitted in the background after each token) and, if non-null, resident [E]
 * (1 for the experts resident at the end). Deterministic. Errors:
 * MOE_ERR_INVALID_ARG for null arrays, shapes outside 1 <= k <= capacity <= E <=
 * 1 << 20 and T >= 0, ids out of range or repeated within a token;
 * MOE_ERR_UNSUPPORTED for an unknown policy. */
typedef enum {
  MOE_MISS_FETCH_ALL = 0,
  MOE_MISS_RULE = 1,
  MOE_MISS_FIRST_CHOICE = 2
} moe_miss_policy;
moe_status moe_miss_replay(const int32_t* topk_idx, const float* topk_gate, int32_t T, int32_t k, int32_t E,
                           int32_t capacity, int32_t policy, float threshold, float admit_beta, float* m,
                           int32_t* sync_fetches, int32_t* bg_fetches, uint8_t* resident);

/* Staged decode: a resident stack of experts behind a slot table.
 * "The Other Half of the Memory Wall: Serving 35B MoEs from SSD with Trained
 * Routing Prediction" (xyznot.com), 重要用語 (glossary): expert indices are mapped
 * through a slot table on the GPU into a fixed set of expert slots (no allocation
 * per step), and the stacked expert tensor is updated in place by rewriting only
 * the slots whose expert changed.
 *
 * moe_stage_experts copies, for i < n, expert experts[i] of `pool` (its gate/up
 * codes and scales, its down codes and scales) into slot slots[i] of `stack`.
 * `stack` is an expert set of the same H, I and codec whose E is its slot count.
 * experts [n] and slots [n] are DEVICE int32 arrays, trusted to lie in [0, pool->E)
 * and [0, stack->E), with distinct slots. All eight weight and scale pointers must
 * be 16-byte aligned. Asynchronous on `stream`.
 *
 * moe_remap_ids writes out[i] = slot_of[idx[i]] for i < n, and -1 for an id
 * outside [0, E) (DEVICE arrays; slot_of [E] holding each resident expert's slot),
 * so a routing can be run on the stack with moe_gather_qmm_forward.
 *
 * moe_layer_forward_staged is moe_layer_forward with the slot table in the
 * kernels' weight addressing: the router ranges over E experts (router_w [E][H]),
 * and the weights of routed expert e are read from slot slot_of[e] of `stack`
 * (DEVICE int32 [E], 4-byte aligned; stack->E is the slot count). Routing
 * outputs are expert ids. A routed expert whose entry lies outside [0, stack->E)
 * is not resident: it contributes nothing (its gate stays as routed; the pages
 * leave the substitute of a missed expert open). For one token the entries are
 * read beside the logits in the gate/up kernel, so the lookup adds no dependent
 * memory read. `ws` holds moe_workspace_bytes(T, E, H, I, k, scheme) bytes.
 *
 * Errors: MOE_ERR_INVALID_ARG for null or misaligned pointers, n < 0, stacks whose
 * H, I or codec differ from the pool's; the layer's errors for the staged layer;
 * MOE_ERR_HIP for a failed launch. */
moe_status moe_stage_experts(const moe_experts* pool, const moe_experts* stack, const int32_t* experts,
                             const int32_t* slots, int32_t n, void* stream);
moe_status moe_remap_ids(const int32_t* idx, int64_t n, const int32_t* slot_of, int32_t E, int32_t* out,
                         void* stream);
moe_status moe_layer_forward_staged(const void* x, int32_t xtype, int32_t T, const float* router_w, int32_t E,
                                    const moe_experts* stack, const int32_t* slot_of, int32_t k, uint32_t flags,
                                    float* y, int32_t* topk_idx_out, float* topk_gate_out, void* ws,
                                    size_t ws_bytes, void* stream);

/* Prerouter head, run at one layer to give the next layer's routing for the
 * next token. "The Other Half of the Memory Wall: Serving 35B MoEs from SSD with
 * Trained Routing Prediction" (xyznot.com), section 手法 (method), "Prerouterヘッド
 * のアーキテクチャ" (prerouter head architecture): the input is the hidden state
 * joined with the top-k one-hot routing vectors of the current and the previous
 * token, H + 2E values, and the head is fc2(erf-gelu(fc1(input))) plus a linear
 * residual path warm-started from the next layer's router. Section 主なアイデア
 * (main ideas), prediction as routing: the head's top-k is used as the routing.
 *
 * Per token t, with f = [x_t ; khot(cur_t) ; khot(prev_t)] (khot(ids): 1 at each of
 * the k ids, 0 elsewhere; all 0 for a NULL array):
 *   a = gelu(w1 f + b1), gelu(z) = z/2 * (1 + erf(z / sqrt 2))   (F values, fp32)
 *   logits_t = w2 a + b2 + wl f                                   (E values, fp32)
 * then moe_route's softmax and top-k on logits_t.
 * Weights, DEVICE fp32 arrays in this layout (16-byte aligned; b1, b2 may be NULL
 * for no bias):
 *   w1 [F][H+2E], b1 [F], w2 [E][F], b2 [E], wl [E][H+2E] (no bias; at warm start
 *   its first H columns are the next layer's router weights).
 * Limits: H and F multiples of 32 in [32, 4096]; E even, in [2, 1024]; k as for
 * moe_route, and the k of cur/prev equals the output k. */
typedef struct moe_prerouter {
  int32_t H, E, F;
  const float* w1;
  const float* b1;
  const float* w2;
  const float* b2;
  const float* wl;
} moe_prerouter;

/* Workspace for moe_prerouter_forward: fc1 activations [T][F], residual-path
 * partial sums and head logits [T][E] each (fp32). Returns 0 for sizes outside
 * the limits. */
size_t moe_prerouter_workspace_bytes(int32_t T, int32_t E, int32_t F);

/*   x:          [T][H] activations of type xtype (16-byte aligned).
 *   cur, prev:  [T][k] int32 routed ids of the current and previous token, or
 *               NULL (a zero vector, e.g. the first token). Ids must lie in
 *               [0, E) and be distinct per token, as moe_route produces them;
 *               they are not checked on the device.
 *   topk_idx, topk_gate: out [T][k], as moe_route's (flags: MOE_FLAG_RENORM);
 *               both NULL to skip the top-k (logits must then be given, e.g.
 *               for moe_experts_from_logits, which runs the top-k itself).
 *   logits:     out [T][E] fp32 head logits (16-byte aligned), or NULL.
 * Errors: MOE_ERR_INVALID_ARG for NULL or misaligned pointers and sizes outside
 * the limits; MOE_ERR_UNSUPPORTED for an unknown xtype or flag;
 * MOE_ERR_WORKSPACE, MOE_ERR_HIP as elsewhere. */
moe_status moe_prerouter_forward(const void* x, int32_t xtype, int32_t T, const moe_prerouter* head,
                                 const int32_t* cur, const int32_t* prev, int32_t k, uint32_t flags,
                                 int32_t* topk_idx, float* topk_gate, float* logits, void* ws, size_t ws_bytes,
                                 void* stream);

/* One layer of prerouted decode (prediction as routing, "The Other Half of the
 * Memory Wall: Serving 35B MoEs from SSD with Trained Routing Prediction"
 * (xyznot.com), section 主なアイデア): moe_experts_from_logits on the logits
 * predicted for this layer, then, when head is not NULL, the next layer's head
 * (moe_prerouter_forward, logits only) on this layer's input, with this layer's
 * routing as the current-token k-hot input and prev_idx as the previous one.
 * For one token on the matvec path (I <= 1024, F <= 1024) both run together in
 * two launches: the head's rows are extra workgroups of the gate/up and down
 * launches. Otherwise the calls run one after the other.
 *   logits:        [T][E] fp32 predicted for this layer (16-byte aligned).
 *   topk_idx_out:  out [T][k], this layer's routing; required with a head (it
 *                  is the next token's prev_idx).
 *   prev_idx:      [T][k] this layer's routing at the previous token, or NULL;
 *                  not the same array as topk_idx_out.
 *   logits_next:   out [T][E] fp32, the next layer's predicted logits (16-byte
 *                  aligned); required with a head. It must not alias `logits`.
 *   ws:            moe_workspace_bytes(T, E, H, I, k, scheme) rounded up to 256,
 *                  plus moe_prerouter_workspace_bytes(T, E, F) with a head.
 * Errors as moe_experts_from_logits and moe_prerouter_forward, and
 * MOE_ERR_INVALID_ARG for a head whose H or E differ from the experts'. */
moe_status moe_prerouted_layer_forward(const void* x, int32_t xtype, int32_t T, const float* logits,
                                       const moe_experts* ex, int32_t k, uint32_t flags, float* y,
                                       int32_t* topk_idx_out, float* topk_gate_out, const moe_prerouter* head,
                                       const int32_t* prev_idx, float* logits_next, void* ws, size_t ws_bytes,
                                       void* stream);

/* Block-quantized linear with an unmerged LoRA delta. "The Other Half of the
 * Memory Wall: Serving 35B MoEs from SSD with Trained Routing Prediction"
 * (xyznot.com), section 手法 (method), "非マージアダプターの実行" (running the
 * unmerged adapter): the layer keeps its quantized base weights and runs the
 * low-rank delta beside them, y = W_q x + (alpha / r) B A x; section よくある質問
 * (FAQ): merged into 4-bit weights and re-quantised, the delta is mostly lost.
 *
 * moe_qweight: one matrix [N][K] in the experts' block format (codes [N][K]
 * bytes for sym8, [N][K/2] for int4; scales [N][K/32] binary16).
 *   y[t][n] = sum_i W_q[n][i] x[t][i] + scale * sum_j B[n][j] (sum_i A[j][i] x[t][i])
 *   x:      [T][K] activations of type xtype (16-byte aligned).
 *   lora_a: [r][K] fp32 (16-byte aligned), lora_b: [N][r] fp32; both ignored when
 *           r == 0 (the plain quantized linear).
 *   scale:  alpha / r.
 *   y:      out [T][N] fp32.
 * Limits: K a multiple of 32 in [32, 4096]; 1 <= N <= 65536; 0 <= r <= 64;
 * 1 <= T <= 65536. `ws` holds moe_qlinear_lora_workspace_bytes(T, r) bytes
 * (u = A x). Errors as elsewhere. */
typedef struct moe_qweight {
  int32_t N, K;
  int32_t scheme;           /* moe_qscheme */
  const void* codes;
  const uint16_t* scales;
} moe_qweight;
size_t moe_qlinear_lora_workspace_bytes(int32_t T, int32_t r);
moe_status moe_qlinear_lora_forward(const void* x, int32_t xtype, int32_t T, const moe_qweight* w,
                                    const float* lora_a, const float* lora_b, int32_t r, float scale, float* y,
                                    void* ws, size_t ws_bytes, void* stream);

/* Benchmark support: the achievable-bandwidth reference. Reads `bytes` bytes
 * (a positive multiple of 16) of the device buffer `buf` once, with coalesced
 * 16-byte non-temporal loads spread over the whole GPU, and writes nothing.
 * It is the plain streaming read that a gathered kernel moving the same bytes
 * is compared with, next to the HBM peak. Errors: MOE_ERR_INVALID_ARG for a
 * null or misaligned buf or a bad size. */
moe_status moe_stream_read(const void* buf, int64_t bytes, void* stream);

/* Static description of a status code. */
const char* moe_status_str(moe_status s);

/* Detail of the last error returned to the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
