/* Host sanitizer run of the oracle (test infrastructure): every oref_* entry
 * point on small seeded shapes of both codecs and all activation types, plus
 * its argument checks, built with -fsanitize=address,undefined. Light property
 * checks only; the pins live in the Python tests. Exit 0 and "ok" on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double urand(void) {
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (double)(rng >> 11) * (1.0 / 9007199254740992.0);
}
static float nrand(void) {
  double u = urand() + 1e-12, v = urand();
  return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); exit(1); } } while (0)

static void* xbuf(int T, int H, int xtype) {
  if (xtype == OREF_F32) {
    float* x = malloc(sizeof(float) * T * H);
    for (int i = 0; i < T * H; ++i) x[i] = nrand();
    return x;
  }
  uint16_t* x = malloc(2 * (size_t)T * H);
  for (int i = 0; i < T * H; ++i) {
    float f = nrand();
    if (xtype == OREF_F16) x[i] = oref_f32_to_f16(f);
    else { uint32_t u; memcpy(&u, &f, 4); x[i] = (uint16_t)(u >> 16); }
  }
  return x;
}

static void one_case(int T, int H, int I, int E, int k, int scheme, int xtype) {
  const int cb = scheme == OREF_SYM8 ? 1 : 2;
  const int64_t ngu = (int64_t)E * 2 * I, nd = (int64_t)E * H;
  float* wgu = malloc(sizeof(float) * ngu * H);
  float* wd = malloc(sizeof(float) * nd * I);
  for (int64_t i = 0; i < ngu * H; ++i) wgu[i] = 0.02f * nrand();
  for (int64_t i = 0; i < nd * I; ++i) wd[i] = 0.02f * nrand();
  uint8_t* cgu = malloc(ngu * H / cb);
  uint16_t* sgu = malloc(2 * ngu * (H / 32));
  uint8_t* cd = malloc(nd * I / cb);
  uint16_t* sd = malloc(2 * nd * (I / 32));
  CHECK(oref_quantize(wgu, ngu, H, scheme, cgu, sgu) == 0);
  CHECK(oref_quantize(wd, nd, I, scheme, cd, sd) == 0);
  float* back = malloc(sizeof(float) * ngu * H);
  CHECK(oref_dequantize(cgu, sgu, ngu, H, scheme, back) == 0);
  float* R = malloc(sizeof(float) * E * H);
  for (int i = 0; i < E * H; ++i) R[i] = 0.05f * nrand();
  void* x = xbuf(T, H, xtype);
  double* lg = malloc(sizeof(double) * T * E);
  CHECK(oref_logits(x, xtype, T, H, R, E, lg) == 0);
  int32_t* idx = malloc(sizeof(int32_t) * T * k);
  float* gate = malloc(sizeof(float) * T * k);
  CHECK(oref_route(x, xtype, T, H, R, E, k, OREF_RENORM, idx, gate) == 0);
  for (int i = 0; i < T * k; ++i) CHECK(idx[i] >= 0 && idx[i] < E);
  float* lgf = malloc(sizeof(float) * T * E);
  for (int i = 0; i < T * E; ++i) lgf[i] = (float)lg[i];
  int32_t* idx2 = malloc(sizeof(int32_t) * T * k);
  float* gate2 = malloc(sizeof(float) * T * k);
  CHECK(oref_topk_logits(lgf, T, E, k, 0, idx2, gate2) == 0);
  int32_t* counts = malloc(4 * E); int32_t* offs = malloc(4 * (E + 1));
  int32_t* perm = malloc(4 * T * k); int32_t* uniq = malloc(4 * E); int32_t nu = 0;
  CHECK(oref_group(idx, T, k, E, counts, offs, perm, uniq, &nu) == 0);
  CHECK(offs[E] == T * k && nu >= 1 && nu <= E);
  oref_experts ex = {E, H, I, scheme, cgu, sgu, cd, sd};
  float* y = malloc(sizeof(float) * T * H);
  float* ys = malloc(sizeof(float) * T * k * H);
  CHECK(oref_gather_forward(x, xtype, T, &ex, k, idx, gate, y) == 0);
  CHECK(oref_gather_forward(x, xtype, T, &ex, k, idx, NULL, ys) == 0);
  float* y2 = malloc(sizeof(float) * T * H);
  CHECK(oref_layer_forward(x, xtype, T, R, &ex, k, OREF_RENORM, y2, NULL, NULL) == 0);
  float* gfull = calloc((size_t)T * E, sizeof(float));
  for (int t = 0; t < T; ++t) for (int s = 0; s < k; ++s) gfull[t * E + idx[t * k + s]] = gate[t * k + s];
  float* yd = malloc(sizeof(float) * T * H);
  CHECK(oref_dense_forward(x, xtype, T, &ex, gfull, yd) == 0);
  for (int t = 0; t < T; ++t) {
    double n2 = 0, mx = 0;
    for (int h = 0; h < H; ++h) { n2 += (double)y[t * H + h] * y[t * H + h]; mx = fmax(mx, fabs(y[t * H + h] - yd[t * H + h])); }
    CHECK(mx <= 1e-5 * sqrt(n2) + 1e-30);
    for (int h = 0; h < H; ++h) CHECK(y[t * H + h] == y2[t * H + h]);
  }
  /* prerouter head with history, then without */
  const int F = 32, D = H + 2 * E;
  float* w1 = malloc(sizeof(float) * F * D); float* b1 = malloc(sizeof(float) * F);
  float* w2 = malloc(sizeof(float) * E * F); float* b2 = malloc(sizeof(float) * E);
  float* wl = malloc(sizeof(float) * E * D);
  for (int i = 0; i < F * D; ++i) w1[i] = 0.05f * nrand();
  for (int i = 0; i < F; ++i) b1[i] = 0.1f * nrand();
  for (int i = 0; i < E * F; ++i) w2[i] = 0.05f * nrand();
  for (int i = 0; i < E; ++i) b2[i] = 0.1f * nrand();
  for (int i = 0; i < E * D; ++i) wl[i] = 0.05f * nrand();
  double* hl = malloc(sizeof(double) * T * E);
  CHECK(oref_prerouter(x, xtype, T, H, E, F, w1, b1, w2, b2, wl, idx, idx2, k, OREF_RENORM, idx2, gate2, hl) == 0);
  CHECK(oref_prerouter(x, xtype, T, H, E, F, w1, NULL, w2, NULL, wl, NULL, NULL, k, 0, idx2, gate2, hl) == 0);
  /* quantized linear with and without a delta */
  const int N = 2 * I, r = 4;
  float* A = malloc(sizeof(float) * r * H); float* B = malloc(sizeof(float) * N * r);
  for (int i = 0; i < r * H; ++i) A[i] = 0.1f * nrand();
  for (int i = 0; i < N * r; ++i) B[i] = 0.1f * nrand();
  float* yl = malloc(sizeof(float) * T * N);
  CHECK(oref_qlinear_lora(x, xtype, T, N, H, scheme, cgu, sgu, A, B, r, 0.5, yl) == 0);
  CHECK(oref_qlinear_lora(x, xtype, T, N, H, scheme, cgu, sgu, NULL, NULL, 0, 0.0, yl) == 0);
  /* planted mistakes run the same loops */
  for (int m = 1; m <= 5; ++m) {
    oref_set_plant(m);
    CHECK(oref_gather_forward(x, xtype, T, &ex, k, idx, gate, y) == 0);
  }
  oref_set_plant(0);
  free(wgu); free(wd); free(cgu); free(sgu); free(cd); free(sd); free(back); free(R); free(x); free(lg);
  free(idx); free(gate); free(lgf); free(idx2); free(gate2); free(counts); free(offs); free(perm); free(uniq);
  free(y); free(ys); free(y2); free(gfull); free(yd); free(w1); free(b1); free(w2); free(b2); free(wl); free(hl);
  free(A); free(B); free(yl);
}

int main(void) {
  /* every 65536 fp16 pattern through both conversions */
  for (uint32_t b = 0; b < 65536; ++b) {
    float f = oref_f16_to_f32((uint16_t)b);
    if (f == f) CHECK(oref_f32_to_f16(f) == (uint16_t)b || (b & 0x7FFF) == 0);
    (void)oref_bf16_to_f32((uint16_t)b);
  }
  static const int shapes[][5] = {{3, 64, 32, 6, 3}, {2, 96, 96, 5, 2}, {1, 256, 128, 16, 4}, {4, 32, 64, 2, 2}};
  for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
    for (int scheme = 0; scheme < 2; ++scheme)
      for (int xt = 0; xt < 3; ++xt)
        one_case(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], shapes[i][4], scheme, xt);
  /* argument checks return errors, never touch memory */
  float w[64];
  uint8_t c[64];
  uint16_t s[4];
  CHECK(oref_quantize(w, 1, 33, OREF_SYM8, c, s) < 0);
  CHECK(oref_quantize(w, 1, 32, 7, c, s) < 0);
  int32_t bad[2] = {0, 9};
  int32_t cn[4], of[5], pe[2], un[4], n;
  CHECK(oref_group(bad, 1, 2, 4, cn, of, pe, un, &n) < 0);
  printf("ok\n");
  return 0;
}
