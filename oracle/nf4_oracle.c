/*
 * nf4_oracle.c -- plain, slow CPU oracle for blockwise NF4/FP4 4-bit weight
 * quantization, double quantization, dequantization and the 4-bit-weight x
 * bf16-activation product.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke entry point and the
 * benchmark's CPU-baseline leg load this library. The product path (the HIP
 * library) shares no code, header, table or constant with it.
 *
 * Sources (web pages about bitsandbytes; cited by title and section):
 *  [NF4 page]   CSDN blog "bitsandbytes 是一个用于高效量化和加载大型语言模型（LLM）
 *               的开源库" (blog.csdn.net/blog_programb/article/details/163192907):
 *               table "数学原理对比" (rows 数值表示 / 量化目标 / 缩放机制 / 零点),
 *               table "实际性能差异" (row 训练稳定性（QLoRA）: double quant), and the
 *               closing notes "补充说明" (fp4 = equal-spaced float like E2M1).
 *  [repo page]  ossradar.top "bitsandbytes-foundation/bitsandbytes": release
 *               notes 0.49.2 (blocksize 64 default, blocksize 32), 0.50.0
 *               (fused 4-bit dequantize + GEMM replacing GEMV and
 *               dequantize + F.linear), 0.50.2 (mask the absmax store).
 *  [usage page] icman.com.cn/news/48546 "bitsandbytes 0.49.2" guide:
 *               "Configuration" (compute dtype: bf16 preferred after 4-bit
 *               dequantization), "Core Usage 1" (quant_type, double quant).
 *
 * Arithmetic conventions: IEEE binary32 with round-to-nearest-even for every
 * stored fp32 value (x86-64 SSE, built with -ffp-contract=off, no fast-math,
 * no flush-to-zero); fp64 where a reference sum or a table derivation needs
 * headroom. bf16 is the upper half of a binary32.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - codebook: quantiles of a standard normal truncated at delta = 929/960,
 *    7 negative levels, an exact 0, 8 positive levels, normalised to [-1, 1];
 *  - normalisation s = RN(x / a), a = block absmax; a = 0 gives s = 0;
 *  - code = nearest codebook value to s; an exact tie goes to the smaller value;
 *  - packing: element 2i in bits 7..4 of byte i, element 2i+1 in bits 3..0,
 *    the pad nibble of an odd-length tensor is 0;
 *  - double quant: symmetric absmax int8 per group of 256 absmax values,
 *    s2 = RN(m / 127), q = clamp(rint(RN(a / s2)), -127, 127), ties to even;
 *  - dequant: a' = a, or RN(q * s2) with double quant; w = RN(c[code] * a');
 *    the bf16 compute-dtype weight is RNE_bf16(w);
 *  - matmul: y[m, n] = sum_k bf16(w[n, k]) * x[m, k] summed in fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR 1

/* ------------------------------------------------------------------ bf16 */

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round a finite binary32 to bf16, ties to even, by exact integer arithmetic:
 * add half an ulp of bf16 minus one, plus the lsb that is kept, then truncate. */
static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint32_t keep_lsb = (u >> 16) & 1u;
  u += 0x7fffu + keep_lsb;
  return (uint16_t)(u >> 16);
}

uint16_t orc_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }
float orc_bf16_to_f32(uint16_t h) { return bf16_to_f32(h); }

/* ------------------------------------------------------------------ fp16 */

/* IEEE binary16 -> binary32, exact: sign, 5-bit exponent (bias 15), 10-bit
 * fraction; exponent 0 holds zero and the subnormals frac * 2^-24. */
static float f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 31, frac = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)frac, -24);
  else if (e == 31) v = frac ? NAN : INFINITY;
  else v = ldexp((double)(1024 + frac), e - 25);
  return (float)(sign ? -v : v); /* exact: at most 11 significant bits */
}

/* binary32 -> binary16, round to nearest, ties to even, by exact arithmetic
 * on the value: the result is the multiple of the binary16 spacing at the
 * input's magnitude (2^-24 for subnormals) nearest to it; magnitudes that
 * round to 2^16 or beyond give infinity. */
static uint16_t f32_to_f16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
  double a = fabs((double)f);
  if (a == 0.0) return sign;
  int ex; /* a = m * 2^ex with m in [0.5, 1) */
  frexp(a, &ex);
  int q = ex - 11 < -24 ? -24 : ex - 11; /* spacing exponent: 11 significant bits */
  double scaled = ldexp(a, -q);          /* exact (power-of-two scaling) */
  double r = floor(scaled);
  double frac = scaled - r; /* exact */
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  double v = ldexp(r, q); /* the rounded magnitude */
  if (v >= 65536.0) return (uint16_t)(sign | 0x7c00u);
  /* encode v: subnormal if below 2^-14 */
  if (v < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)ldexp(v, 24));
  int e2;
  double m = frexp(v, &e2); /* v = m 2^e2, m in [0.5, 1) */
  uint16_t exp_field = (uint16_t)(e2 - 1 + 15);
  uint16_t frac_field = (uint16_t)(ldexp(m, 11) - 1024.0);
  return (uint16_t)(sign | (exp_field << 10) | frac_field);
}

uint16_t orc_f32_to_f16(float f) { return f32_to_f16_rne(f); }
float orc_f16_to_f32(uint16_t h) { return f16_to_f32(h); }

/* Element types of tensors passed as raw bits. */
#define ORC_BF16 0
#define ORC_FP32 1
#define ORC_FP16 2

/* Element i of a typed tensor as a binary32 value (exact for every type). */
static float elem_f32(const void *t, int dtype, int64_t i) {
  if (dtype == ORC_BF16) return bf16_to_f32(((const uint16_t *)t)[i]);
  if (dtype == ORC_FP16) return f16_to_f32(((const uint16_t *)t)[i]);
  return ((const float *)t)[i];
}

/* ------------------------------------------------- standard normal quantile */

/* Upper tail Q(z) = P(Z > z) = erfc(z / sqrt 2) / 2, using the C library's erfc. */
static double upper_tail(double z) { return 0.5 * erfc(z / sqrt(2.0)); }

/* The z >= 0 with Q(z) = q, for 0 < q <= 1/2, by bisection: Q is strictly
 * decreasing, so halving [0, 40] until the two ends are neighbouring doubles
 * brackets the root to the last bit that the library erfc resolves. */
static double upper_tail_root(double q) {
  double lo = 0.0, hi = 40.0;
  for (int it = 0; it < 4000; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (upper_tail(mid) > q)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

/* Phi^{-1}(p): slow and obviously correct. For p >= 1/2 the upper tail is
 * 1 - p (exact in fp64 there); for p < 1/2 the lower tail p is used directly
 * through the symmetry Phi(-z) = Q(z), so no precision is lost to 1 - p. */
double orc_norm_ppf(double p) {
  if (!(p > 0.0 && p < 1.0)) return NAN;
  if (p >= 0.5) return upper_tail_root(1.0 - p);
  return -upper_tail_root(p);
}

/* --------------------------------------------------------------- codebooks */

#define ORC_NF4 0
#define ORC_FP4 1

/* NF4 truncation point delta = 1 - (1/32 + 1/30) / 2 = 929/960 (a reading:
 * the NF4 page gives only the resulting values -1, -0.697, -0.525, 0, ...). */
static const double NF4_DELTA = 929.0 / 960.0;

/* NF4 codebook, index = 4-bit code, ascending [NF4 page, table 数学原理对比,
 * row 数值表示: 16 values from a truncated normal, all in [-1, 1], containing 0].
 * Negative side: 7 equal steps in probability from 1/2 to delta; positive side:
 * 8 equal steps; each level is the normal quantile divided by Phi^{-1}(delta)
 * so that the extreme levels are exactly -1 and +1. */
static void nf4_values_f64(double v[16]) {
  double zmax = orc_norm_ppf(NF4_DELTA);
  for (int j = 7; j >= 1; --j) /* codes 0..6 */
    v[7 - j] = -orc_norm_ppf(0.5 + (NF4_DELTA - 0.5) * (double)j / 7.0) / zmax;
  v[7] = 0.0; /* code 7: exact zero [NF4 page, row 零点] */
  for (int j = 1; j <= 8; ++j) /* codes 8..15 */
    v[7 + j] = orc_norm_ppf(0.5 + (NF4_DELTA - 0.5) * (double)j / 8.0) / zmax;
  v[0] = -1.0; /* j = 7 gives exactly -zmax / zmax; written out for clarity */
  v[15] = 1.0;
}

/* FP4 value of a nibble [NF4 page, notes 补充说明: fp4 is an equal-spaced-style
 * float like E2M1]: bit 3 = sign, bits 2..1 = exponent, bit 0 = mantissa, with
 * the E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} divided by 6 so the largest
 * magnitude is 1, as for NF4. */
static double fp4_value_f64(int nib) {
  int sign = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
  double mag = (e == 0) ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
  double v = mag / 6.0;
  return sign ? -v : v;
}

/* fp32 codebook indexed by the 4-bit code. */
int orc_codebook(int quant_type, float out[16]) {
  if (quant_type == ORC_NF4) {
    double v[16];
    nf4_values_f64(v);
    for (int i = 0; i < 16; ++i) out[i] = (float)v[i];
    return ORC_OK;
  }
  if (quant_type == ORC_FP4) {
    for (int i = 0; i < 16; ++i) out[i] = (float)fp4_value_f64(i);
    return ORC_OK;
  }
  return ORC_ERR;
}

/* The candidate codes in ascending order of value. FP4 nibble 8 (-0) is left
 * out, so a zero input always gets nibble 0. */
static int sorted_candidates(int quant_type, float vals[16], int codes[16]) {
  if (orc_codebook(quant_type, vals) != ORC_OK) return 0;
  int n = 0;
  for (int c = 0; c < 16; ++c) {
    if (quant_type == ORC_FP4 && c == 8) continue;
    codes[n++] = c;
  }
  /* insertion sort by value (ascending); plain and small */
  for (int i = 1; i < n; ++i) {
    int c = codes[i], j = i - 1;
    while (j >= 0 && vals[codes[j]] > vals[c]) {
      codes[j + 1] = codes[j];
      --j;
    }
    codes[j + 1] = c;
  }
  return n;
}

/* Nearest codebook value to s [NF4 page, row 量化目标: minimise the squared
 * quantization error]. Distances are taken in fp64, where s - c is exact for
 * every |s| >= 2^-29 (and tinier s are nearest to 0 by a wide margin). Scanning
 * in ascending order with a strict '<' sends an exact tie to the smaller value. */
static int nearest_code(float s, const float vals[16], const int cand[16], int ncand) {
  int best = cand[0];
  double bd = fabs((double)s - (double)vals[cand[0]]);
  for (int i = 1; i < ncand; ++i) {
    double d = fabs((double)s - (double)vals[cand[i]]);
    if (d < bd) {
      bd = d;
      best = cand[i];
    }
  }
  return best;
}

int orc_nearest_code(int quant_type, float s) {
  float vals[16];
  int cand[16];
  int nc = sorted_candidates(quant_type, vals, cand);
  if (nc == 0) return -1;
  return nearest_code(s, vals, cand, nc);
}

/* ---------------------------------------------------------------- quantize */

/* Blockwise quantization [NF4 page, row 缩放机制: each block gets its own scale
 * max|x|; values are normalised into [-1, 1] and mapped to the nearest of the
 * 16 code values]. Blocks are bs consecutive elements of the flattened tensor
 * (the release notes' 1-D blocksize 64/128/...); the last block may be short
 * and its absmax covers only its real elements [repo page, 0.50.2: mask the
 * absmax store]. The input is bf16, fp16 or fp32 (dtype), each element taken
 * as its exact binary32 value. Outputs: packed[ceil(n/2)], absmax[ceil(n/bs)]. */
int orc_quantize_typed(const void *w, int dtype, int64_t n, int bs, int quant_type,
                       uint8_t *packed, float *absmax) {
  float vals[16];
  int cand[16];
  int nc = sorted_candidates(quant_type, vals, cand);
  if (nc == 0 || bs <= 0 || n < 0) return ORC_ERR;
  if (dtype != ORC_BF16 && dtype != ORC_FP16 && dtype != ORC_FP32) return ORC_ERR;
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(elem_f32(w, dtype, i))) return ORC_ERR;
  int64_t nb = (n + bs - 1) / bs;
  for (int64_t i = 0; i < (n + 1) / 2; ++i) packed[i] = 0;
  for (int64_t b = 0; b < nb; ++b) {
    int64_t lo = b * bs, hi = lo + bs < n ? lo + bs : n;
    float a = 0.0f;
    for (int64_t i = lo; i < hi; ++i) {
      float v = fabsf(elem_f32(w, dtype, i));
      if (v > a) a = v;
    }
    absmax[b] = a;
    for (int64_t i = lo; i < hi; ++i) {
      float x = elem_f32(w, dtype, i);
      float s = (a == 0.0f) ? 0.0f : x / a; /* binary32 division, RN */
      int code = nearest_code(s, vals, cand, nc);
      if (i % 2 == 0)
        packed[i / 2] |= (uint8_t)(code << 4);
      else
        packed[i / 2] |= (uint8_t)code;
    }
  }
  return ORC_OK;
}

int orc_quantize(const uint16_t *w, int64_t n, int bs, int quant_type, uint8_t *packed,
                 float *absmax) {
  return orc_quantize_typed(w, ORC_BF16, n, bs, quant_type, packed, absmax);
}

/* ------------------------------------------------------------ double quant */

/* Second-level quantization of the fp32 block scales to 8 bits [NF4 page,
 * table 实际性能差异, row 训练稳定性（QLoRA）: the NF4 scales are quantized again
 * with INT8 to shrink the metadata]. Groups of bs2 consecutive absmax values;
 * per group m = max a, s2 = RN(m / 127), q = clamp(rint(RN(a / s2)), -127, 127).
 * rintf rounds half to even in the default rounding mode. */
int orc_double_quant(const float *absmax, int64_t nb, int bs2, int8_t *q, float *s2) {
  if (bs2 <= 0 || nb < 0) return ORC_ERR;
  int64_t ng = (nb + bs2 - 1) / bs2;
  for (int64_t g = 0; g < ng; ++g) {
    int64_t lo = g * bs2, hi = lo + bs2 < nb ? lo + bs2 : nb;
    float m = 0.0f;
    for (int64_t i = lo; i < hi; ++i) {
      float v = fabsf(absmax[i]);
      if (v > m) m = v;
    }
    if (m == 0.0f) {
      s2[g] = 0.0f;
      for (int64_t i = lo; i < hi; ++i) q[i] = 0;
      continue;
    }
    float scale = m / 127.0f;
    s2[g] = scale;
    for (int64_t i = lo; i < hi; ++i) {
      float r = rintf(absmax[i] / scale);
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      q[i] = (int8_t)r;
    }
  }
  return ORC_OK;
}

/* Mean-centred variant of the second level (a reading: the NF4 page says only
 * that the scales are quantized again to INT8; centring each group on its
 * mean lets the int8 codes use both signs). Per group of bs2 consecutive
 * absmax values a_0 .. a_{L-1} (L = bs2, or fewer in the last group):
 *   S  = pairwise binary32 sum of the group padded with zeros to bs2 values
 *        (adjacent pairs first: level by level, element i of a level is
 *        element 2i plus element 2i+1 of the level below), mu = RN(S / L);
 *   D  = max_i |RN(a_i - mu)|; s2 = RN(D / 127), or 0 when D = 0;
 *   q_i = clamp(rint(RN(RN(a_i - mu) / s2)), -127, 127), or 0 when s2 = 0.
 * Stores q (int8), s2 and mu (fp32 each). The dequantized scale is
 * a' = RN(RN(q * s2) + mu). bs2 must be a power of two (at most 4096). */
int orc_double_quant_centred(const float *absmax, int64_t nb, int bs2, int8_t *q, float *s2,
                             float *offset) {
  if (bs2 <= 0 || bs2 > 4096 || (bs2 & (bs2 - 1)) != 0 || nb < 0) return ORC_ERR;
  float buf[4096];
  int64_t ng = (nb + bs2 - 1) / bs2;
  for (int64_t g = 0; g < ng; ++g) {
    int64_t lo = g * bs2, hi = lo + bs2 < nb ? lo + bs2 : nb;
    int64_t L = hi - lo;
    for (int i = 0; i < bs2; ++i) buf[i] = (lo + i < hi) ? absmax[lo + i] : 0.0f;
    for (int w = bs2; w > 1; w >>= 1)
      for (int i = 0; i < w / 2; ++i) buf[i] = buf[2 * i] + buf[2 * i + 1];
    float mu = buf[0] / (float)L;
    float D = 0.0f;
    for (int64_t i = lo; i < hi; ++i) {
      float d = fabsf(absmax[i] - mu);
      if (d > D) D = d;
    }
    offset[g] = mu;
    if (D == 0.0f) {
      s2[g] = 0.0f;
      for (int64_t i = lo; i < hi; ++i) q[i] = 0;
      continue;
    }
    float scale = D / 127.0f;
    s2[g] = scale;
    for (int64_t i = lo; i < hi; ++i) {
      float r = rintf((absmax[i] - mu) / scale);
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      q[i] = (int8_t)r;
    }
  }
  return ORC_OK;
}

/* ---------------------------------------------------------------- dequant */

static int code_at(const uint8_t *packed, int64_t i) {
  uint8_t byte = packed[i / 2];
  return (i % 2 == 0) ? (byte >> 4) : (byte & 15);
}

/* Effective block scale a' of block b: the stored fp32 absmax; with double
 * quant RN(q * s2) of the int8 code and its group's fp32 scale; with the
 * mean-centred variant (offset != NULL) RN(RN(q * s2) + mu). */
static float block_scale(int64_t b, const float *absmax, const int8_t *q, const float *s2,
                         const float *offset, int bs2) {
  if (q == NULL) return absmax[b];
  float t = (float)q[b] * s2[b / bs2];
  if (offset == NULL) return t;
  return t + offset[b / bs2];
}

/* Dequantize to the fp32 value w = RN(c[code] * a') and, for each 16-bit
 * output given, to RNE_bf16(w) and RNE_fp16(w) [usage page, Configuration:
 * the compute dtype is the precision used after 4-bit dequantization].
 * q == NULL selects the plain fp32 absmax; otherwise q/s2 (and the group
 * offsets when given) are used. */
int orc_dequantize_typed(const uint8_t *packed, int64_t n, int bs, int quant_type,
                         const float *absmax, const int8_t *q, const float *s2,
                         const float *offset, int bs2, float *out_f32, uint16_t *out_bf16,
                         uint16_t *out_f16) {
  float vals[16];
  if (orc_codebook(quant_type, vals) != ORC_OK || bs <= 0 || n < 0) return ORC_ERR;
  if (q == NULL && absmax == NULL) return ORC_ERR;
  for (int64_t i = 0; i < n; ++i) {
    float ap = block_scale(i / bs, absmax, q, s2, offset, bs2);
    float w = vals[code_at(packed, i)] * ap; /* binary32 product, RN */
    if (out_f32) out_f32[i] = w;
    if (out_bf16) out_bf16[i] = f32_to_bf16_rne(w);
    if (out_f16) out_f16[i] = f32_to_f16_rne(w);
  }
  return ORC_OK;
}

int orc_dequantize(const uint8_t *packed, int64_t n, int bs, int quant_type, const float *absmax,
                   const int8_t *q, const float *s2, int bs2, float *out_f32, uint16_t *out_bf16) {
  return orc_dequantize_typed(packed, n, bs, quant_type, absmax, q, s2, NULL, bs2, out_f32,
                              out_bf16, NULL);
}

/* ----------------------------------------------------------------- matmul */

/* y[m, n] = sum_k Wc[n, k] * x[m, k] in fp64, where Wc is the bf16 compute-dtype
 * weight (row-major [N, K]) and x the bf16 activations (row-major [M, K]).
 * Each product of two bf16 values is exact in fp64; the sum runs in k order.
 * [repo page, 0.50.0: the 4-bit GEMV / fused dequantize + GEMM compute the
 * product of the activations with the dequantized weight.] */
int orc_matmul_bf16(const uint16_t *x, const uint16_t *wc, int64_t M, int64_t N, int64_t K,
                    double *y) {
  if (M < 0 || N < 0 || K < 0) return ORC_ERR;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k)
        acc += (double)bf16_to_f32(wc[n * K + k]) * (double)bf16_to_f32(x[m * K + k]);
      y[m * N + n] = acc;
    }
  return ORC_OK;
}

/* The same sum for a list of (m, n) output positions only, for shapes whose
 * full product is too slow here. */
int orc_matmul_bf16_sampled(const uint16_t *x, const uint16_t *wc, int64_t K, const int64_t *ms,
                            const int64_t *ns, int64_t count, double *y) {
  if (K < 0 || count < 0) return ORC_ERR;
  for (int64_t i = 0; i < count; ++i) {
    double acc = 0.0;
    const uint16_t *wr = wc + ns[i] * K, *xr = x + ms[i] * K;
    for (int64_t k = 0; k < K; ++k) acc += (double)bf16_to_f32(wr[k]) * (double)bf16_to_f32(xr[k]);
    y[i] = acc;
  }
  return ORC_OK;
}

/* Whole decode product straight from the quantized form: dequantize row n to
 * bf16 (as orc_dequantize does) and take its fp64 dot product with each x row. */
int orc_gemv_quantized(const uint16_t *x, int64_t M, const uint8_t *packed, int64_t N, int64_t K,
                       int bs, int quant_type, const float *absmax, const int8_t *q,
                       const float *s2, int bs2, double *y) {
  float vals[16];
  if (orc_codebook(quant_type, vals) != ORC_OK || bs <= 0 || M < 0 || N < 0 || K < 0)
    return ORC_ERR;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t m = 0; m < M; ++m) y[m * N + n] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      int64_t i = n * K + k;
      float ap = block_scale(i / bs, absmax, q, s2, NULL, bs2);
      float w = vals[code_at(packed, i)] * ap;
      double wc = (double)bf16_to_f32(f32_to_bf16_rne(w));
      for (int64_t m = 0; m < M; ++m) y[m * N + n] += wc * (double)bf16_to_f32(x[m * K + k]);
    }
  }
  return ORC_OK;
}

/* y[m, n] = sum_k Wc[n, k] * x[m, k] in fp64 for operands of one element type
 * (bf16, fp16 or fp32 -- the compute dtype; every product of two such values
 * is exact in fp64), summed in k order. */
int orc_matmul_typed(const void *x, const void *wc, int dtype, int64_t M, int64_t N, int64_t K,
                     double *y) {
  if (M < 0 || N < 0 || K < 0) return ORC_ERR;
  if (dtype != ORC_BF16 && dtype != ORC_FP16 && dtype != ORC_FP32) return ORC_ERR;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k)
        acc += (double)elem_f32(wc, dtype, n * K + k) * (double)elem_f32(x, dtype, m * K + k);
      y[m * N + n] = acc;
    }
  return ORC_OK;
}

/* The decode product straight from the quantized form in a compute dtype:
 * each weight is dequantized (block_scale, then RN(c * a')), rounded to the
 * compute dtype (bf16 or fp16 RNE; fp32 kept as is), and its fp64 product
 * with the activation (of the same dtype) summed in k order. */
int orc_gemv_quantized_typed(const void *x, int dtype, int64_t M, const uint8_t *packed,
                             int64_t N, int64_t K, int bs, int quant_type, const float *absmax,
                             const int8_t *q, const float *s2, const float *offset, int bs2,
                             double *y) {
  float vals[16];
  if (orc_codebook(quant_type, vals) != ORC_OK || bs <= 0 || M < 0 || N < 0 || K < 0)
    return ORC_ERR;
  if (dtype != ORC_BF16 && dtype != ORC_FP16 && dtype != ORC_FP32) return ORC_ERR;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t m = 0; m < M; ++m) y[m * N + n] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      int64_t i = n * K + k;
      float ap = block_scale(i / bs, absmax, q, s2, offset, bs2);
      float w = vals[code_at(packed, i)] * ap;
      double wc;
      if (dtype == ORC_BF16) wc = (double)bf16_to_f32(f32_to_bf16_rne(w));
      else if (dtype == ORC_FP16) wc = (double)f16_to_f32(f32_to_f16_rne(w));
      else wc = (double)w;
      for (int64_t m = 0; m < M; ++m) y[m * N + n] += wc * (double)elem_f32(x, dtype, m * K + k);
    }
  }
  return ORC_OK;
}

/* Elementwise conversion of n values between the element types (via the
 * exact binary32 value; to bf16 / fp16 with RNE). */
int orc_convert(const void *in, int in_dtype, int64_t n, void *out, int out_dtype) {
  if (n < 0) return ORC_ERR;
  for (int64_t i = 0; i < n; ++i) {
    float f = elem_f32(in, in_dtype, i);
    if (out_dtype == ORC_BF16) ((uint16_t *)out)[i] = f32_to_bf16_rne(f);
    else if (out_dtype == ORC_FP16) ((uint16_t *)out)[i] = f32_to_f16_rne(f);
    else if (out_dtype == ORC_FP32) ((float *)out)[i] = f;
    else return ORC_ERR;
  }
  return ORC_OK;
}

/* ----------------------------------------------------- host-thread harness */

/* The decode product split over T host threads by whole output rows, each
 * thread running the sequential code above on its share, so the result is
 * bitwise that of the single-threaded call. Used only to time the oracle on
 * all host cores. */

struct orc_gemv_job {
  const void *x;
  int dtype;
  int64_t M, N0, N1, K;
  const uint8_t *packed;
  int bs, quant_type, bs2;
  const float *absmax, *s2, *offset;
  const int8_t *q;
  double *y; /* [M, N1 - N0] rows of this job, row stride N1 - N0 */
  int rc;
};

static void *orc_gemv_worker(void *arg) {
  struct orc_gemv_job *j = (struct orc_gemv_job *)arg;
  /* the rows [N0, N1) of W are a weight of N1 - N0 rows starting at element
   * N0 * K; its blocks start at block N0 * K / bs (K % bs == 0) */
  int64_t e0 = j->N0 * j->K, b0 = e0 / j->bs;
  const float *a = j->absmax ? j->absmax + b0 : NULL;
  const int8_t *q = j->q ? j->q + b0 : NULL;
  /* group-aligned shares only (the caller splits on multiples of bs2 blocks) */
  const float *s2 = j->s2 ? j->s2 + b0 / j->bs2 : NULL;
  const float *off = j->offset ? j->offset + b0 / j->bs2 : NULL;
  j->rc = orc_gemv_quantized_typed(j->x, j->dtype, j->M, j->packed + e0 / 2, j->N1 - j->N0, j->K,
                                   j->bs, j->quant_type, a, q, s2, off, j->bs2, j->y);
  return NULL;
}

/* orc_gemv_quantized_typed over T threads; rows are split on multiples of
 * `row_align` rows (whole double-quant groups when row_align * K / bs is a
 * multiple of bs2). y is [M, N]. */
int orc_gemv_quantized_threads(const void *x, int dtype, int64_t M, const uint8_t *packed,
                               int64_t N, int64_t K, int bs, int quant_type, const float *absmax,
                               const int8_t *q, const float *s2, const float *offset, int bs2,
                               double *y, int threads, int64_t row_align) {
  if (threads < 1 || threads > 1024 || row_align < 1 || M < 0 || N < 0) return ORC_ERR;
  if (K % bs != 0 || (q != NULL && ((row_align * K / bs) % bs2) != 0)) return ORC_ERR;
  struct orc_gemv_job jobs[1024];
  pthread_t tid[1024];
  double *parts[1024];
  int64_t units = (N + row_align - 1) / row_align;
  int nt = threads < units ? threads : (int)(units > 0 ? units : 1);
  for (int t = 0; t < nt; ++t) {
    int64_t u0 = units * t / nt, u1 = units * (t + 1) / nt;
    int64_t n0 = u0 * row_align, n1 = u1 * row_align < N ? u1 * row_align : N;
    parts[t] = (double *)malloc(sizeof(double) * (size_t)(M * (n1 - n0) + 1));
    jobs[t] = (struct orc_gemv_job){x, dtype, M, n0, n1, K, packed, bs, quant_type, bs2,
                                    absmax, s2, offset, q, parts[t], 0};
    pthread_create(&tid[t], NULL, orc_gemv_worker, &jobs[t]);
  }
  int rc = ORC_OK;
  for (int t = 0; t < nt; ++t) {
    pthread_join(tid[t], NULL);
    if (jobs[t].rc != ORC_OK) rc = ORC_ERR;
    int64_t w = jobs[t].N1 - jobs[t].N0;
    for (int64_t m = 0; m < M; ++m)
      for (int64_t n = 0; n < w; ++n) y[m * N + jobs[t].N0 + n] = parts[t][m * w + n];
    free(parts[t]);
  }
  return rc;
}
