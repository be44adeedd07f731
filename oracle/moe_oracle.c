/*
 * moe_oracle.c — plain CPU oracle for the routed, block-quantized MoE expert layer.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may load it. It shares nothing with the GPU
 * library. Page citations use the keys defined in moe_oracle.h:
 *   [LR] "QwenのMoEルーターを観測してホットエキスパートを先読みしても速くならなかった" (lilting.ch)
 *   [QK] "鳴かぬなら、カスタムカーネル、ほととぎす" (qiita.com, john-rocky)
 *   [MW] "The Other Half of the Memory Wall: Serving 35B MoEs from SSD with
 *        Trained Routing Prediction" (xyznot.com)
 *
 * Precision: activations are upcast exactly; weights are code * scale, which is
 * exact in fp32; every sum runs in fp64 and results are rounded to fp32 once.
 * The only integer decision taken on floating point, the top-k choice, is
 * taken on fp32-rounded logits, the precision the router's gate linear
 * produces [LR "hooking the router"].
 *
 * OpenMP parallelises only loops whose iterations are independent (one output
 * element each); each element's sum keeps its sequential order, so the results
 * do not depend on the thread count.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int32_t g_plant = 0;

void oref_set_plant(int32_t mistake) { g_plant = mistake; }

int32_t oref_num_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}

void oref_set_num_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ---------------- number formats (IEEE 754-2008 binary16, bfloat16) ---------------- */

/* fp32 -> binary16, round to nearest, ties to even. Finite values at or above
 * 65520 (half-way past the largest finite 65504) round to infinity. */
uint16_t oref_f32_to_f16(float f) {
  uint32_t bits;
  memcpy(&bits, &f, 4);
  const uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
  const double a = fabs((double)f);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);           /* a in [2^(e2-1), 2^e2) */
  int ex = e2 - 1;          /* unbiased exponent of a */
  if (ex < -14) ex = -14;   /* subnormals share the spacing 2^-24 */
  const double spacing = ldexp(1.0, ex - 10);
  double n = nearbyint(a / spacing);  /* a / spacing is exact; default rounding is ties-to-even */
  uint32_t m = (uint32_t)n;           /* in [0, 2048] */
  if (m == 2048u) { ex += 1; m = 1024u; }
  if (ex > 15) return (uint16_t)(sign | 0x7C00u);
  if (m < 1024u) return (uint16_t)(sign | m); /* subnormal (only possible when ex == -14) */
  return (uint16_t)(sign | (uint32_t)((ex + 15) << 10) | (m - 1024u));
}

float oref_f16_to_f32(uint16_t h) {
  const int s = (h >> 15) & 1;
  const int ex = (h >> 10) & 0x1F;
  const int m = h & 0x3FF;
  double v;
  if (ex == 0) v = ldexp((double)m, -24);
  else if (ex == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), ex - 25);
  return (float)(s ? -v : v);
}

/* bfloat16 is the upper half of an fp32 bit pattern. */
float oref_bf16_to_f32(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

static double x_elem(const void* x, int32_t xtype, int64_t i) {
  switch (xtype) {
    case OREF_F32: return (double)((const float*)x)[i];
    case OREF_F16: return (double)oref_f16_to_f32(((const uint16_t*)x)[i]);
    default:       return (double)oref_bf16_to_f32(((const uint16_t*)x)[i]);
  }
}

/* ---------------- block quantisation [QK §6: sym8, per-K-block-32] ---------------- */

static int qmax_of(int32_t scheme) { return scheme == OREF_SYM8 ? 127 : 7; }

int oref_quantize(const float* w, int64_t rows, int32_t K, int32_t scheme,
                  uint8_t* codes, uint16_t* scales) {
  if (!w || !codes || !scales || rows < 0 || K <= 0 || K % 32) return -1;
  if (scheme != OREF_SYM8 && scheme != OREF_INT4) return -2;
  const int qmax = qmax_of(scheme);
  const int nb = K / 32;
  #pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int b = 0; b < nb; ++b) {
      const float* blk = w + r * K + (int64_t)b * 32;
      float amax = 0.0f;
      for (int j = 0; j < 32; ++j) {
        const float a = fabsf(blk[j]);
        if (a > amax) amax = a;
      }
      uint16_t s16 = oref_f32_to_f16(amax / (float)qmax);
      if ((s16 & 0x7FFFu) == 0x7C00u) s16 = (uint16_t)((s16 & 0x8000u) | 0x7BFFu); /* saturate */
      scales[r * nb + b] = s16;
      const float s = oref_f16_to_f32(s16);
      for (int j = 0; j < 32; ++j) {
        int q = 0;
        if (s != 0.0f) {
          float t = rintf(blk[j] / s);
          if (t > (float)qmax) t = (float)qmax;
          if (t < (float)-qmax) t = (float)-qmax;
          q = (int)t;
        }
        const int64_t kk = (int64_t)b * 32 + j;
        if (scheme == OREF_SYM8) {
          codes[r * K + kk] = (uint8_t)(int8_t)q;
        } else {
          uint8_t* byte = codes + r * (K / 2) + kk / 2;
          const uint8_t nib = (uint8_t)(q & 0xF);
          if ((kk & 1) == 0) *byte = (uint8_t)((*byte & 0xF0u) | nib);
          else               *byte = (uint8_t)((*byte & 0x0Fu) | (uint8_t)(nib << 4));
        }
      }
    }
  }
  return 0;
}

/* Code of element j of a row (sign-extended). */
static int code_at(const uint8_t* row_codes, int32_t scheme, int32_t j) {
  if (scheme == OREF_SYM8) return (int)(int8_t)row_codes[j];
  const uint8_t byte = row_codes[j / 2];
  int low_is_even = (g_plant == 4) ? 0 : 1;
  const int nib = ((j & 1) == (low_is_even ? 0 : 1)) ? (byte & 0xF) : (byte >> 4);
  return nib >= 8 ? nib - 16 : nib;
}

/* Dequantised weight w[row][j] = code * scale (exact in fp32). */
static float weight_at(const uint8_t* codes, const uint16_t* scales, int32_t scheme,
                       int64_t row, int32_t K, int32_t j) {
  const int64_t row_bytes = scheme == OREF_SYM8 ? K : K / 2;
  const int nb = K / 32;
  int b = j / 32;
  if (g_plant == 5) b = (b + 1) % nb;
  const float s = oref_f16_to_f32(scales[row * nb + b]);
  return (float)code_at(codes + row * row_bytes, scheme, j) * s;
}

int oref_dequantize(const uint8_t* codes, const uint16_t* scales, int64_t rows,
                    int32_t K, int32_t scheme, float* w) {
  if (!codes || !scales || !w || rows < 0 || K <= 0 || K % 32) return -1;
  if (scheme != OREF_SYM8 && scheme != OREF_INT4) return -2;
  #pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t j = 0; j < K; ++j) w[r * K + j] = weight_at(codes, scales, scheme, r, K, j);
  return 0;
}

/* ---------------- router [LR "hooking the router"] ---------------- */

int oref_logits(const void* x, int32_t xtype, int32_t T, int32_t H,
                const float* R, int32_t E, double* logits) {
  if (!x || !R || !logits || T < 0 || H <= 0 || E <= 0) return -1;
  if (xtype < OREF_F32 || xtype > OREF_BF16) return -2;
  #pragma omp parallel for collapse(2) schedule(static)
  for (int32_t t = 0; t < T; ++t)
    for (int32_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int32_t h = 0; h < H; ++h)
        acc += x_elem(x, xtype, (int64_t)t * H + h) * (double)R[(int64_t)e * H + h];
      logits[(int64_t)t * E + e] = acc;
    }
  return 0;
}

/* Softmax over the E logits of one token, then the top k [LR "hooking the
 * router"]: k rounds of "largest fp32-rounded logit not yet taken, lowest id on
 * ties"; each chosen expert's probability, divided by the sum over the k when
 * flags has OREF_RENORM. Returns nonzero when out of memory. */
static int softmax_topk_row(const double* l, int32_t E, int32_t k, uint32_t flags,
                            int32_t* idx, float* gate) {
  /* softmax over all E experts, in fp64 (max subtracted first) */
  double mx = l[0];
  for (int32_t e = 1; e < E; ++e) if (l[e] > mx) mx = l[e];
  double* p = (double*)malloc(sizeof(double) * (size_t)E);
  char* taken = (char*)calloc((size_t)E, 1);
  if (!p || !taken) { free(p); free(taken); return 1; }
  double z = 0.0;
  for (int32_t e = 0; e < E; ++e) { p[e] = exp(l[e] - mx); z += p[e]; }
  for (int32_t e = 0; e < E; ++e) p[e] /= z;
  double psum = 0.0;
  for (int32_t s = 0; s < k; ++s) {
    int32_t best = -1;
    float bv = 0.0f;
    for (int32_t e = 0; e < E; ++e) {
      if (taken[e]) continue;
      const float v = (float)l[e];
      if (best < 0 || v > bv) { best = e; bv = v; }
    }
    taken[best] = 1;
    idx[s] = best;
    psum += p[best];
  }
  for (int32_t s = 0; s < k; ++s) {
    const double ps = p[idx[s]];
    gate[s] = (float)((flags & OREF_RENORM) ? ps / psum : ps);
  }
  free(p);
  free(taken);
  return 0;
}

int oref_route(const void* x, int32_t xtype, int32_t T, int32_t H,
               const float* R, int32_t E, int32_t k, uint32_t flags,
               int32_t* idx, float* gate) {
  if (!x || !R || !idx || !gate || T < 0 || H <= 0 || E <= 0 || k < 1 || k > E) return -1;
  double* lg = (double*)malloc(sizeof(double) * ((size_t)T * (size_t)E + 1));
  if (!lg) return -3;
  int rc = oref_logits(x, xtype, T, H, R, E, lg);
  if (rc) { free(lg); return rc; }
  int fail = 0;
  #pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < T; ++t)
    if (softmax_topk_row(lg + (int64_t)t * E, E, k, flags, idx + (int64_t)t * k, gate + (int64_t)t * k))
      fail = 1;
  free(lg);
  return fail ? -3 : 0;
}

/* The router's softmax and top-k on given fp32 logits [T][E] (as oref_route
 * after its gate linear). */
int oref_topk_logits(const float* logits, int32_t T, int32_t E, int32_t k, uint32_t flags, int32_t* idx,
                     float* gate) {
  if (!logits || !idx || !gate || T < 0 || E <= 0 || k < 1 || k > E) return -1;
  int fail = 0;
  #pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < T; ++t) {
    double* l = (double*)malloc(sizeof(double) * (size_t)E);
    if (!l) { fail = 1; continue; }
    for (int32_t e = 0; e < E; ++e) l[e] = (double)logits[(int64_t)t * E + e];
    if (softmax_topk_row(l, E, k, flags, idx + (int64_t)t * k, gate + (int64_t)t * k)) fail = 1;
    free(l);
  }
  return fail ? -3 : 0;
}

/* ---------------- prerouter head ---------------- */

/* erf-form GELU: z * Phi(z), Phi the standard normal CDF, written with erf
 * [MW "Prerouterヘッドのアーキテクチャ" (prerouter head architecture)]. */
static double gelu_erf(double z) { return 0.5 * z * (1.0 + erf(z / sqrt(2.0))); }

int oref_prerouter(const void* x, int32_t xtype, int32_t T, int32_t H, int32_t E, int32_t F,
                   const float* w1, const float* b1, const float* w2, const float* b2,
                   const float* wl, const int32_t* cur, const int32_t* prev, int32_t k,
                   uint32_t flags, int32_t* idx, float* gate, double* logits) {
  if (!x || !w1 || !w2 || !wl || !idx || !gate || !logits || T < 0 || H <= 0 || E <= 0 || F <= 0 ||
      k < 1 || k > E) return -1;
  if (xtype < OREF_F32 || xtype > OREF_BF16) return -2;
  const int32_t D = H + 2 * E;
  int bad = 0;
  for (int64_t i = 0; i < (int64_t)T * k; ++i) {
    if (cur && (cur[i] < 0 || cur[i] >= E)) bad = 1;
    if (prev && (prev[i] < 0 || prev[i] >= E)) bad = 1;
  }
  if (bad) return -1;
  int fail = 0;
  #pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < T; ++t) {
    /* the input feature: hidden state, then the k-hot routing vector of the
     * current token, then that of the previous token (dim = d_model + 2E) */
    double* f = (double*)calloc((size_t)D, sizeof(double));
    double* a = (double*)malloc(sizeof(double) * (size_t)F);
    if (!f || !a) { free(f); free(a); fail = 1; continue; }
    for (int32_t i = 0; i < H; ++i) f[i] = x_elem(x, xtype, (int64_t)t * H + i);
    for (int32_t s = 0; s < k; ++s) {
      if (cur) f[H + cur[(int64_t)t * k + s]] = 1.0;
      if (prev) f[H + E + prev[(int64_t)t * k + s]] = 1.0;
    }
    /* a = erf-gelu(fc1(f)) */
    for (int32_t j = 0; j < F; ++j) {
      double z = b1 ? (double)b1[j] : 0.0;
      for (int32_t i = 0; i < D; ++i) z += (double)w1[(int64_t)j * D + i] * f[i];
      a[j] = gelu_erf(z);
    }
    /* head = fc2(a) + l(f), l the bias-free linear residual path */
    double* l = logits + (int64_t)t * E;
    for (int32_t e = 0; e < E; ++e) {
      double acc = b2 ? (double)b2[e] : 0.0;
      for (int32_t j = 0; j < F; ++j) acc += (double)w2[(int64_t)e * F + j] * a[j];
      for (int32_t i = 0; i < D; ++i) acc += (double)wl[(int64_t)e * D + i] * f[i];
      l[e] = acc;
    }
    free(f);
    free(a);
    if (softmax_topk_row(l, E, k, flags, idx + (int64_t)t * k, gate + (int64_t)t * k)) fail = 1;
  }
  return fail ? -3 : 0;
}

/* ---------------- quantized linear with an unmerged LoRA delta ---------------- */

/* [MW] section 手法, "非マージアダプターの実行" (running the unmerged adapter): the
 * layer keeps its quantized base weights and runs the low-rank delta beside them,
 * y = W_q x + (alpha / r) B A x, with W_q = code * scale [QK section 6]. */
int oref_qlinear_lora(const void* x, int32_t xtype, int32_t T, int32_t N, int32_t K, int32_t scheme,
                      const uint8_t* codes, const uint16_t* scales, const float* A, const float* B, int32_t r,
                      double scale, float* y) {
  if (!x || !codes || !scales || !y || T < 0 || N <= 0 || K <= 0 || K % 32 || r < 0) return -1;
  if (r > 0 && (!A || !B)) return -1;
  if (xtype < OREF_F32 || xtype > OREF_BF16) return -2;
  if (scheme != OREF_SYM8 && scheme != OREF_INT4) return -2;
  int fail = 0;
  #pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < T; ++t) {
    double* u = (double*)malloc(sizeof(double) * ((size_t)r + 1));
    if (!u) { fail = 1; continue; }
    /* u = A x_t, the adapter's down projection */
    for (int32_t j = 0; j < r; ++j) {
      double acc = 0.0;
      for (int32_t i = 0; i < K; ++i) acc += (double)A[(int64_t)j * K + i] * x_elem(x, xtype, (int64_t)t * K + i);
      u[j] = acc;
    }
    for (int32_t n = 0; n < N; ++n) {
      double base = 0.0;
      for (int32_t i = 0; i < K; ++i)
        base += (double)weight_at(codes, scales, scheme, n, K, i) * x_elem(x, xtype, (int64_t)t * K + i);
      double delta = 0.0;
      for (int32_t j = 0; j < r; ++j) delta += (double)B[(int64_t)n * r + j] * u[j];
      y[(int64_t)t * N + n] = (float)(base + scale * delta);
    }
    free(u);
  }
  return fail ? -3 : 0;
}

/* ---------------- token-by-expert grouping ---------------- */

int oref_group(const int32_t* idx, int32_t T, int32_t k, int32_t E,
               int32_t* counts, int32_t* offsets, int32_t* perm,
               int32_t* uniq, int32_t* n_uniq) {
  if (!idx || !counts || !offsets || !perm || !uniq || !n_uniq || T < 0 || k < 1 || E < 1) return -1;
  const int64_t n = (int64_t)T * k;
  for (int64_t f = 0; f < n; ++f) if (idx[f] < 0 || idx[f] >= E) return -1;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < n; ++f) counts[idx[f]] += 1;
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int64_t pos = 0;
  for (int32_t e = 0; e < E; ++e)
    for (int64_t f = 0; f < n; ++f)
      if (idx[f] == e) perm[pos++] = (int32_t)f;
  int32_t u = 0;
  for (int32_t e = 0; e < E; ++e) if (counts[e] > 0) uniq[u++] = e;
  *n_uniq = u;
  return 0;
}

/* ---------------- expert FFN [QK §4, §7] ---------------- */

static int check_experts(const oref_experts* ex) {
  if (!ex || !ex->w_gate_up || !ex->s_gate_up || !ex->w_down || !ex->s_down) return -1;
  if (ex->E < 1 || ex->H < 32 || ex->I < 32 || ex->H % 32 || ex->I % 32) return -1;
  if (ex->scheme != OREF_SYM8 && ex->scheme != OREF_INT4) return -2;
  return 0;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Row n of the SwiGLU activation of expert e on token x:
 * u_gate = W_gu[e][n] . x, u_up = W_gu[e][I + n] . x, h = silu(u_gate) * u_up. */
static double gate_up_swiglu_row(const oref_experts* ex, int32_t e, const double* xt, int32_t n) {
  const int32_t H = ex->H, I = ex->I;
  const int64_t row0 = (int64_t)e * 2 * I;
  double ug = 0.0, uu = 0.0;
  for (int32_t j = 0; j < H; ++j) {
    ug += (double)weight_at(ex->w_gate_up, ex->s_gate_up, ex->scheme, row0 + n, H, j) * xt[j];
    uu += (double)weight_at(ex->w_gate_up, ex->s_gate_up, ex->scheme, row0 + I + n, H, j) * xt[j];
  }
  return (g_plant == 2) ? silu(uu) * ug : silu(ug) * uu;
}

/* Row m of the down projection of expert e: W_d[e][m] . h. */
static double down_row(const oref_experts* ex, int32_t e, const double* h, int32_t m) {
  const int32_t I = ex->I;
  const int64_t row = (int64_t)e * ex->H + m;
  double acc = 0.0;
  for (int32_t j = 0; j < I; ++j)
    acc += (double)weight_at(ex->w_down, ex->s_down, ex->scheme, row, I, j) * h[j];
  return acc;
}

int oref_gather_forward(const void* x, int32_t xtype, int32_t T,
                        const oref_experts* ex, int32_t k,
                        const int32_t* idx, const float* gate, float* y) {
  int rc = check_experts(ex);
  if (rc) return rc;
  if (!x || !idx || !y || T < 0 || k < 1) return -1;
  if (xtype < OREF_F32 || xtype > OREF_BF16) return -2;
  for (int64_t f = 0; f < (int64_t)T * k; ++f) if (idx[f] < 0 || idx[f] >= ex->E) return -1;
  const int32_t H = ex->H, I = ex->I;
  const int64_t TK = (int64_t)T * k;
  double* xd = (double*)malloc(sizeof(double) * ((size_t)T * (size_t)H + 1));
  double* h = (double*)malloc(sizeof(double) * ((size_t)TK * (size_t)I + 1));
  double* ys = (double*)malloc(sizeof(double) * ((size_t)TK * (size_t)H + 1));
  if (!xd || !h || !ys) { free(xd); free(h); free(ys); return -3; }
  for (int64_t i = 0; i < (int64_t)T * H; ++i) xd[i] = x_elem(x, xtype, i);
  /* gate/up share the token; SwiGLU per slot */
  #pragma omp parallel for collapse(2) schedule(static)
  for (int64_t f = 0; f < TK; ++f)
    for (int32_t n = 0; n < I; ++n)
      h[f * I + n] = gate_up_swiglu_row(ex, idx[f], xd + (f / k) * H, n);
  /* down projection per slot, each on its own activation */
  #pragma omp parallel for collapse(2) schedule(static)
  for (int64_t f = 0; f < TK; ++f)
    for (int32_t m = 0; m < H; ++m) {
      const int64_t fh = (g_plant == 1) ? (f / k) * k : f;
      ys[f * H + m] = down_row(ex, idx[f], h + fh * I, m);
    }
  /* gate-weighted combine, in slot order */
  if (gate) {
    #pragma omp parallel for collapse(2) schedule(static)
    for (int32_t t = 0; t < T; ++t)
      for (int32_t m = 0; m < H; ++m) {
        double acc = 0.0;
        for (int32_t s = 0; s < k; ++s) {
          const int64_t f = (int64_t)t * k + s;
          const double g = (g_plant == 3) ? 1.0 : (double)gate[f];
          acc += g * ys[f * H + m];
        }
        y[(int64_t)t * H + m] = (float)acc;
      }
  } else {
    for (int64_t i = 0; i < TK * H; ++i) y[i] = (float)ys[i];
  }
  free(xd);
  free(h);
  free(ys);
  return 0;
}

int oref_layer_forward(const void* x, int32_t xtype, int32_t T, const float* R,
                       const oref_experts* ex, int32_t k, uint32_t flags, float* y,
                       int32_t* idx_out, float* gate_out) {
  int rc = check_experts(ex);
  if (rc) return rc;
  if (!y || T < 0 || k < 1 || k > ex->E) return -1;
  int32_t* idx = idx_out ? idx_out : (int32_t*)malloc(sizeof(int32_t) * (size_t)T * (size_t)k + 1);
  float* gate = gate_out ? gate_out : (float*)malloc(sizeof(float) * (size_t)T * (size_t)k + 1);
  if (!idx || !gate) rc = -3;
  if (!rc) rc = oref_route(x, xtype, T, ex->H, R, ex->E, k, flags, idx, gate);
  if (!rc) rc = oref_gather_forward(x, xtype, T, ex, k, idx, gate, y);
  if (!idx_out) free(idx);
  if (!gate_out) free(gate);
  return rc;
}

int oref_dense_forward(const void* x, int32_t xtype, int32_t T,
                       const oref_experts* ex, const float* gate_full, float* y) {
  int rc = check_experts(ex);
  if (rc) return rc;
  if (!x || !gate_full || !y || T < 0) return -1;
  if (xtype < OREF_F32 || xtype > OREF_BF16) return -2;
  const int32_t H = ex->H, I = ex->I, E = ex->E;
  const int64_t TE = (int64_t)T * E;
  double* xd = (double*)malloc(sizeof(double) * ((size_t)T * (size_t)H + 1));
  double* h = (double*)malloc(sizeof(double) * ((size_t)TE * (size_t)I + 1));
  if (!xd || !h) { free(xd); free(h); return -3; }
  for (int64_t i = 0; i < (int64_t)T * H; ++i) xd[i] = x_elem(x, xtype, i);
  /* every expert on every token, whatever its gate */
  #pragma omp parallel for collapse(2) schedule(static)
  for (int64_t te = 0; te < TE; ++te)
    for (int32_t n = 0; n < I; ++n)
      h[te * I + n] = gate_up_swiglu_row(ex, (int32_t)(te % E), xd + (te / E) * H, n);
  #pragma omp parallel for collapse(2) schedule(static)
  for (int32_t t = 0; t < T; ++t)
    for (int32_t m = 0; m < H; ++m) {
      double acc = 0.0;
      for (int32_t e = 0; e < E; ++e) {
        const int64_t te = (int64_t)t * E + e;
        acc += (double)gate_full[te] * down_row(ex, e, h + te * I, m);
      }
      y[(int64_t)t * H + m] = (float)acc;
    }
  free(xd);
  free(h);
  return 0;
}
