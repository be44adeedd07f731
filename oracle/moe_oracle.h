/*
 * moe_oracle.h — plain CPU oracle for the routed, block-quantized MoE expert layer.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load this library. The GPU library
 * shares no code, header, table or helper with it.
 *
 * What it computes is the plain definition, written out with no blocking,
 * fusion or reordering: dequantise every weight exactly, then run the expert
 * FFNs densely in fp64 and round the results to fp32.
 *
 * Pages cited (title, then the section):
 *   [LR] "QwenのMoEルーターを観測してホットエキスパートを先読みしても速くならなかった"
 *        (lilting.ch). Sections: "ルーターをフックする" (hooking the router),
 *        "事前ウォームアップとmmapキャッシュを比べる" (the stacked expert array and gather_qmm).
 *   [QK] "鳴かぬなら、カスタムカーネル、ほととぎす" (qiita.com, john-rocky).
 *        Sections: §1 (what MoE buys), §4 (custom kernel gather_qmm),
 *        §6 (quality check), §7 (pitfalls).
 *   [MW] "The Other Half of the Memory Wall: Serving 35B MoEs from SSD with
 *        Trained Routing Prediction" (xyznot.com). Section 手法 (method),
 *        "Prerouterヘッドのアーキテクチャ" (prerouter head architecture) and
 *        "非マージアダプターの実行" (running the unmerged adapter).
 *
 * Conventions:
 *   - All pointers are host pointers, owned by the caller, never retained.
 *   - Shapes are row-major and C-contiguous.
 *   - Functions return 0 on success and a negative value when an argument is
 *     out of range; they never abort.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Activation element types. */
enum { OREF_F32 = 0, OREF_F16 = 1, OREF_BF16 = 2 };
/* Weight codecs: [QK §6] symmetric linear int8 in blocks of 32 along K ("sym8"),
 * and its 4-bit analogue [QK §3, §7] with codes in [-7, 7]. */
enum { OREF_SYM8 = 0, OREF_INT4 = 1 };
/* Route flags: bit 0 renormalises the k gates so they sum to one. */
enum { OREF_RENORM = 1u };

/* IEEE-754 binary16 / bfloat16 conversions (round to nearest, ties to even). */
uint16_t oref_f32_to_f16(float f);
float    oref_f16_to_f32(uint16_t h);
float    oref_bf16_to_f32(uint16_t h);

/* Quantise w[rows][K] (fp32) to codes + one fp16 scale per 32 consecutive K
 * elements of a row [QK §6].
 *   sym8: codes[rows][K]   int8 bytes,      scales[rows][K/32]
 *   int4: codes[rows][K/2] two codes a byte, low nibble = even K index.
 * Per block: s = fp16(amax / qmax) (qmax 127 or 7, the division in fp32),
 * q = clamp(rint(w / s), -qmax, qmax) in fp32, and q = 0 when s == 0.
 * A scale that would round past the largest finite fp16 saturates to it.
 * K must be a positive multiple of 32. */
int oref_quantize(const float* w, int64_t rows, int32_t K, int32_t scheme,
                  uint8_t* codes, uint16_t* scales);

/* w[rows][K] = code * scale, exact in fp32. */
int oref_dequantize(const uint8_t* codes, const uint16_t* scales, int64_t rows,
                    int32_t K, int32_t scheme, float* w);

/* Router logits [LR "hooking the router", first step: the gate linear]:
 * logits[t][e] = sum_h x[t][h] * R[e][h], accumulated in fp64. */
int oref_logits(const void* x, int32_t xtype, int32_t T, int32_t H,
                const float* R, int32_t E, double* logits);

/* Router [LR "hooking the router"]: logits, softmax, top-k.
 * idx[t][0..k-1]: experts by descending fp32-rounded logit, ties to the lower
 * expert id. gate[t][s]: softmax probability of idx[t][s] (fp64), divided by
 * the sum over the k chosen when flags has OREF_RENORM. */
int oref_route(const void* x, int32_t xtype, int32_t T, int32_t H,
               const float* R, int32_t E, int32_t k, uint32_t flags,
               int32_t* idx, float* gate);

/* oref_route's softmax and top-k on given fp32 logits [T][E]. */
int oref_topk_logits(const float* logits, int32_t T, int32_t E, int32_t k, uint32_t flags, int32_t* idx,
                     float* gate);

/* Prerouter head [MW "prerouter head architecture"], per token t:
 *   f = [x_t ; khot(cur_t) ; khot(prev_t)]   (H + 2E values; khot(ids) has a 1
 *       at each of the k ids and 0 elsewhere, all 0 when the array is NULL)
 *   a = gelu(w1 f + b1),  gelu(z) = z/2 * (1 + erf(z / sqrt 2))   (F values)
 *   logits_t = w2 a + b2 + wl f                                   (E values)
 * then the router's softmax and top-k (as oref_route) on logits_t.
 * Shapes: w1 [F][H+2E], b1 [F] or NULL, w2 [E][F], b2 [E] or NULL,
 * wl [E][H+2E] (the linear residual path, no bias); cur, prev [T][k] ids in
 * [0, E) or NULL. Outputs idx [T][k], gate [T][k], logits [T][E] (fp64). */
int oref_prerouter(const void* x, int32_t xtype, int32_t T, int32_t H, int32_t E, int32_t F,
                   const float* w1, const float* b1, const float* w2, const float* b2,
                   const float* wl, const int32_t* cur, const int32_t* prev, int32_t k,
                   uint32_t flags, int32_t* idx, float* gate, double* logits);

/* Quantized linear with an unmerged LoRA delta [MW "非マージアダプターの実行"]:
 * y[t][n] = sum_i W_q[n][i] x[t][i] + scale * sum_j B[n][j] (sum_i A[j][i] x[t][i]),
 * W_q = code * scale of the codec (codes [N][K] or [N][K/2] for int4, scales
 * [N][K/32]), A [r][K], B [N][r] fp32, scale = alpha / r. r = 0 (A, B unused)
 * is the plain quantized linear. Sums in fp64, y rounded to fp32 once. */
int oref_qlinear_lora(const void* x, int32_t xtype, int32_t T, int32_t N, int32_t K, int32_t scheme,
                      const uint8_t* codes, const uint16_t* scales, const float* A, const float* B, int32_t r,
                      double scale, float* y);

/* Token-by-expert grouping of the T*k flat assignments f = t*k + s:
 * counts[e], offsets[E+1] (exclusive prefix sum), perm[T*k] = the flat ids
 * ordered by expert, then by f; uniq[] = experts with counts > 0, ascending;
 * *n_uniq = their number. */
int oref_group(const int32_t* idx, int32_t T, int32_t k, int32_t E,
               int32_t* counts, int32_t* offsets, int32_t* perm,
               int32_t* uniq, int32_t* n_uniq);

/* Packed experts: the stacked (experts, out, in) array of [LR "warm-up vs
 * mmap cache"] with gate and up concatenated along "out".
 *   w_gate_up: [E][2I][H] codes (rows 0..I-1 gate, I..2I-1 up), scales [E][2I][H/32]
 *   w_down:    [E][H][I]  codes,                                 scales [E][H][I/32]
 * For int4 the innermost dimension holds two codes a byte. */
typedef struct {
  int32_t E, H, I, scheme;
  const uint8_t*  w_gate_up;
  const uint16_t* s_gate_up;
  const uint8_t*  w_down;
  const uint16_t* s_down;
} oref_experts;

/* Gathered expert layer [QK §4, §7]: for each token t and slot s, with
 * e = idx[t][s]: u = W_gu[e] x_t; h = silu(u[0:I]) * u[I:2I] (silu(z) =
 * z / (1 + exp(-z))); ys = W_d[e] h (each slot on its own h).
 * With gate != NULL: y[t][H] = sum_s gate[t][s] * ys, in slot order.
 * With gate == NULL: y[t][s][H] = ys (per-slot outputs).
 * idx entries must lie in [0, E). */
int oref_gather_forward(const void* x, int32_t xtype, int32_t T,
                        const oref_experts* ex, int32_t k,
                        const int32_t* idx, const float* gate, float* y);

/* Whole layer: oref_route then oref_gather_forward. idx_out/gate_out may be NULL. */
int oref_layer_forward(const void* x, int32_t xtype, int32_t T, const float* R,
                       const oref_experts* ex, int32_t k, uint32_t flags, float* y,
                       int32_t* idx_out, float* gate_out);

/* Dense check form: y[t] = sum over all E experts of gate_full[t][e] * FFN_e(x_t),
 * evaluating every expert, including those whose gate is zero. */
int oref_dense_forward(const void* x, int32_t xtype, int32_t T,
                       const oref_experts* ex, const float* gate_full, float* y);

/* Test hook: plants a known mistake in oref_gather_forward so tests can show
 * that their pins and tolerances reject it. 0 = none (default);
 * 1 = every slot's down projection takes slot 0's activation;
 * 2 = gate and up halves swapped; 3 = gates ignored (each slot weighted 1);
 * 4 = int4 nibble order swapped; 5 = scale of block j taken from block j+1 (wraps). */
void oref_set_plant(int32_t mistake);

/* Number of OpenMP threads the oracle's loops use (1 when built without OpenMP). */
int32_t oref_num_threads(void);
/* Sets that number (n > 0; ignored without OpenMP). Results do not depend on
 * it: the loops split independent outputs only. */
void oref_set_num_threads(int32_t n);

#ifdef __cplusplus
}
#endif
#endif
