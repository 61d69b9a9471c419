/*
 * oracle_sanitize_main.c -- drives every entry point of the CPU oracle
 * (oracle/nf4_oracle.c) once on small seeded inputs, so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitized.py)
 * sees each code path: ragged lengths and last blocks, every element type,
 * both double-quant modes, all-zero blocks, and the threaded decode product.
 * Exit status 0 when every call returns success and the light consistency
 * checks below hold; the sanitizers abort on their own findings.
 *
 * Test infrastructure: it links the oracle only, never the HIP library.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define BF16 0
#define FP32 1
#define FP16 2

double orc_norm_ppf(double p);
int orc_codebook(int quant_type, float out[16]);
int orc_nearest_code(int quant_type, float s);
int orc_quantize_typed(const void *w, int dtype, int64_t n, int bs, int quant_type,
                       uint8_t *packed, float *absmax);
int orc_quantize(const uint16_t *w, int64_t n, int bs, int quant_type, uint8_t *packed,
                 float *absmax);
int orc_double_quant(const float *absmax, int64_t nb, int bs2, int8_t *q, float *s2);
int orc_double_quant_centred(const float *absmax, int64_t nb, int bs2, int8_t *q, float *s2,
                             float *mu);
int orc_dequantize_typed(const uint8_t *packed, int64_t n, int bs, int quant_type,
                         const float *absmax, const int8_t *q, const float *s2,
                         const float *offset, int bs2, float *out_f32, uint16_t *out_bf16,
                         uint16_t *out_f16);
int orc_dequantize(const uint8_t *packed, int64_t n, int bs, int quant_type, const float *absmax,
                   const int8_t *q, const float *s2, int bs2, float *out_f32, uint16_t *out_bf16);
int orc_gemv_quantized(const uint16_t *x, int64_t M, const uint8_t *packed, int64_t N, int64_t K,
                       int bs, int quant_type, const float *absmax, const int8_t *q,
                       const float *s2, int bs2, double *y);
int orc_matmul_typed(const void *x, const void *wc, int dtype, int64_t M, int64_t N, int64_t K,
                     double *y);
int orc_gemv_quantized_typed(const void *x, int dtype, int64_t M, const uint8_t *packed,
                             int64_t N, int64_t K, int bs, int quant_type, const float *absmax,
                             const int8_t *q, const float *s2, const float *offset, int bs2,
                             double *y);
int orc_convert(const void *in, int in_dtype, int64_t n, void *out, int out_dtype);
int orc_gemv_quantized_threads(const void *x, int dtype, int64_t M, const uint8_t *packed,
                               int64_t N, int64_t K, int bs, int quant_type, const float *absmax,
                               const int8_t *q, const float *s2, const float *offset, int bs2,
                               double *y, int threads, int64_t row_align);

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double uniform(void) {  /* xorshift64*, in (0, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return ((rng * 0x2545f4914f6cdd1dull) >> 11) * (1.0 / 9007199254740992.0) + 1e-17;
}
static float normal(void) { return (float)(sqrt(-2.0 * log(uniform())) * cos(6.283185307179586 * uniform())); }

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main(void) {
  enum { N = 37, K = 192, M = 3, NK = N * K };
  float cb[16];
  CHECK(orc_codebook(0, cb) == 0 && orc_codebook(1, cb) == 0);
  CHECK(fabs(orc_norm_ppf(0.5)) < 1e-12);
  CHECK(orc_nearest_code(0, 1.0f) == 15 && orc_nearest_code(0, -1.0f) == 0);

  /* weights: N(0, 0.02^2) in fp32, an all-zero block, then bf16 / fp16 copies */
  float *wf = malloc(sizeof(float) * NK);
  for (int i = 0; i < NK; ++i) wf[i] = 0.02f * normal();
  for (int i = 64; i < 128; ++i) wf[i] = 0.0f;
  uint16_t *wb = malloc(2 * NK), *wh = malloc(2 * NK);
  CHECK(orc_convert(wf, FP32, NK, wb, BF16) == 0);
  CHECK(orc_convert(wf, FP32, NK, wh, FP16) == 0);

  const int bss[] = {32, 64, 128};
  for (int qt = 0; qt < 2; ++qt)
    for (int bi = 0; bi < 3; ++bi) {
      const int bs = bss[bi];
      for (int64_t n = NK - 33; n <= NK; n += 33) {  /* ragged and whole */
        const int64_t nb = (n + bs - 1) / bs;
        uint8_t *packed = malloc((size_t)(n + 1) / 2);
        float *absmax = malloc(sizeof(float) * (size_t)nb);
        CHECK(orc_quantize(wb, n, bs, qt, packed, absmax) == 0);
        uint8_t *p2 = malloc((size_t)(n + 1) / 2);
        float *a2 = malloc(sizeof(float) * (size_t)nb);
        CHECK(orc_quantize_typed(wh, FP16, n, bs, qt, p2, a2) == 0);
        CHECK(orc_quantize_typed(wf, FP32, n, bs, qt, p2, a2) == 0);
        /* both double-quant modes, group size 256 (more blocks than one group) */
        int8_t *q = malloc((size_t)nb);
        float *s2 = malloc(sizeof(float) * (size_t)((nb + 255) / 256));
        float *mu = malloc(sizeof(float) * (size_t)((nb + 255) / 256));
        CHECK(orc_double_quant(absmax, nb, 256, q, s2) == 0);
        float *out = malloc(sizeof(float) * (size_t)n);
        uint16_t *ob = malloc(2 * (size_t)n), *oh = malloc(2 * (size_t)n);
        CHECK(orc_dequantize(packed, n, bs, qt, absmax, NULL, NULL, 256, out, ob) == 0);
        for (int64_t i = 64; i < 128 && i < n; ++i) CHECK(out[i] == 0.0f);
        CHECK(orc_dequantize(packed, n, bs, qt, NULL, q, s2, 256, out, ob) == 0);
        CHECK(orc_double_quant_centred(absmax, nb, 256, q, s2, mu) == 0);
        CHECK(orc_dequantize_typed(packed, n, bs, qt, NULL, q, s2, mu, 256, out, ob, oh) == 0);
        free(out); free(ob); free(oh); free(q); free(s2); free(mu);
        free(p2); free(a2); free(packed); free(absmax);
      }
    }

  /* products: x [M, K] in each dtype against the whole [N, K] weight */
  {
    const int bs = 64;
    const int64_t nb = NK / bs;
    uint8_t *packed = malloc(NK / 2);
    float *absmax = malloc(sizeof(float) * nb);
    int8_t *q = malloc(nb);
    float *s2 = malloc(sizeof(float) * ((nb + 255) / 256));
    CHECK(orc_quantize(wb, NK, bs, 0, packed, absmax) == 0);
    CHECK(orc_double_quant(absmax, nb, 256, q, s2) == 0);
    float *xf = malloc(sizeof(float) * M * K);
    for (int i = 0; i < M * K; ++i) xf[i] = normal();
    uint16_t *xb = malloc(2 * M * K), *xh = malloc(2 * M * K);
    CHECK(orc_convert(xf, FP32, M * K, xb, BF16) == 0);
    CHECK(orc_convert(xf, FP32, M * K, xh, FP16) == 0);
    double *y1 = malloc(sizeof(double) * M * N), *y2 = malloc(sizeof(double) * M * N);
    double *y3 = malloc(sizeof(double) * M * N);
    CHECK(orc_gemv_quantized(xb, M, packed, N, K, bs, 0, NULL, q, s2, 256, y1) == 0);
    CHECK(orc_gemv_quantized_typed(xb, BF16, M, packed, N, K, bs, 0, NULL, q, s2, NULL, 256,
                                   y2) == 0);
    CHECK(memcmp(y1, y2, sizeof(double) * M * N) == 0);
    /* row_align 4: 4 rows x 3 blocks = 12 blocks, not whole groups of 256 -> refused */
    CHECK(orc_gemv_quantized_threads(xb, BF16, M, packed, N, K, bs, 0, NULL, q, s2, NULL, 256, y3,
                                     3, 4) != 0);
    /* without double quant any alignment works: bitwise the single-threaded sums */
    CHECK(orc_gemv_quantized_typed(xb, BF16, M, packed, N, K, bs, 0, absmax, NULL, NULL, NULL,
                                   256, y2) == 0);
    CHECK(orc_gemv_quantized_threads(xb, BF16, M, packed, N, K, bs, 0, absmax, NULL, NULL, NULL,
                                     256, y3, 3, 4) == 0);
    CHECK(memcmp(y2, y3, sizeof(double) * M * N) == 0);
    float *wc = malloc(sizeof(float) * NK);
    uint16_t *wcb = malloc(2 * NK), *wch = malloc(2 * NK);
    CHECK(orc_dequantize_typed(packed, NK, bs, 0, absmax, NULL, NULL, NULL, 256, wc, wcb, wch) ==
          0);
    CHECK(orc_matmul_typed(xb, wcb, BF16, M, N, K, y3) == 0);
    CHECK(memcmp(y2, y3, sizeof(double) * M * N) == 0);
    CHECK(orc_matmul_typed(xh, wch, FP16, M, N, K, y3) == 0);
    CHECK(orc_matmul_typed(xf, wc, FP32, M, N, K, y3) == 0);
    CHECK(orc_gemv_quantized_typed(xf, FP32, M, packed, N, K, bs, 0, absmax, NULL, NULL, NULL, 256,
                                   y2) == 0);
    CHECK(memcmp(y2, y3, sizeof(double) * M * N) == 0);
    free(packed); free(absmax); free(q); free(s2); free(xf); free(xb); free(xh);
    free(y1); free(y2); free(y3); free(wc); free(wcb); free(wch);
  }
  free(wf); free(wb); free(wh);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle sanitize run: ok\n");
  return 0;
}
