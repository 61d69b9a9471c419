/*
 * nf4.h -- C ABI of libnf4: blockwise NF4/FP4 4-bit weight quantization and the
 * dequantize-fused 4-bit-weight x bf16-activation product on AMD Instinct
 * MI355X (gfx950).
 *
 * What is computed follows the bitsandbytes pages:
 *  [NF4 page]   CSDN blog "bitsandbytes 是一个用于高效量化和加载大型语言模型（LLM）
 *               的开源库": table 数学原理对比 (codebook, nearest-code objective,
 *               per-block max|x| scale, exact zero), table 实际性能差异 row
 *               训练稳定性（QLoRA） (double quantization: the scales quantized
 *               again to INT8), closing notes 补充说明 (fp4 ~ E2M1).
 *  [repo page]  ossradar.top "bitsandbytes-foundation/bitsandbytes", release
 *               notes 0.49.2 (default blocksize 64; blocksize 32), 0.50.0 (4-bit
 *               GEMV; fused 4-bit dequantize + GEMM), 0.50.2 (the absmax store of
 *               a partial block is masked).
 *  [usage page] icman.com.cn/news/48546 (bitsandbytes 0.49.2 guide),
 *               "Configuration" and "Core Usage 1": quant_type nf4|fp4,
 *               use_double_quant, compute dtype bf16 (the dtype the 4-bit weight
 *               is dequantized to before the matmul).
 *
 * Conventions common to every entry point
 *  - All tensor arguments are DEVICE pointers to caller-owned memory on the
 *    current HIP device. The library never allocates, frees or keeps a pointer
 *    after a call returns. Outputs must not alias inputs.
 *  - Every compute call is asynchronous on `stream` (a hipStream_t; NULL = the
 *    default stream) and returns after the launches are queued. Faults inside a
 *    kernel surface at the caller's next synchronisation.
 *  - Arguments are validated before anything is launched; on any error the call
 *    returns a non-zero status and writes nothing.
 *  - bf16 tensors are passed as raw 16-bit patterns (upper half of a binary32).
 *  - Inputs must be finite; NaN/Inf inputs give unspecified codes.
 *  - Every device pointer must be 16-byte aligned (NF4_ERR_MISALIGNED).
 *  - n == 0 (or M == 0 / N == 0 for the products) is a valid no-op.
 *  - The device must be gfx950 (NF4_ERR_UNSUPPORTED otherwise); with no HIP
 *    device at all the calls return NF4_ERR_DEVICE.
 *  - Stateless apart from per-device constant tables built on first use, so
 *    calls from several host threads are safe. No C++ exception crosses the ABI.
 *
 * Storage of one quantized tensor of n elements (flattened row-major)
 *  - blocks of `blocksize` consecutive elements; nb = ceil(n / blocksize);
 *  - packed  uint8[ceil(n/2)]: element 2i in bits 7..4 of byte i, element 2i+1
 *            in bits 3..0; an odd n leaves the last low nibble 0;
 *  - absmax  float[nb]: max |x| over the block's real elements;
 *  - with double quantization, groups of `blocksize2` consecutive absmax values:
 *    absmax_q int8[nb] and absmax_scale float[ceil(nb/blocksize2)];
 *  - NF4 codes are ranks in the ascending 16-value codebook (code 7 is 0);
 *    FP4 codes are E2M1 nibbles (bit 3 sign, bits 2..1 exponent, bit 0
 *    mantissa) of the E2M1 magnitudes divided by 6.
 * A weight matrix W of N rows (output features) and K columns (input features)
 * is stored as the flattened [N, K] row-major tensor, n = N*K, so blocks run
 * along K; the products require K % blocksize == 0.
 */
#ifndef NF4_H
#define NF4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NF4_ABI_VERSION 1

typedef enum nf4_status {
  NF4_OK = 0,
  NF4_ERR_INVALID_ARGUMENT = 1, /* NULL pointer, negative size, bad enum, shape mismatch */
  NF4_ERR_UNSUPPORTED = 2,      /* valid request this library does not implement, or not gfx950 */
  NF4_ERR_MISALIGNED = 3,       /* a device pointer is not 16-byte aligned */
  NF4_ERR_DEVICE = 4            /* no HIP device, or a HIP call / launch failed */
} nf4_status;

typedef enum nf4_quant_type { NF4_QUANT_NF4 = 0, NF4_QUANT_FP4 = 1 } nf4_quant_type;

typedef enum nf4_dtype { NF4_DTYPE_BF16 = 0, NF4_DTYPE_FP32 = 1 } nf4_dtype;

/* Descriptor of one quantized tensor. The pointers are device pointers owned by
 * the caller; `absmax` is read when double_quant == 0, `absmax_q` and
 * `absmax_scale` when double_quant == 1. Mirrors the pages' configuration
 * fields (quant_type, use_double_quant) plus the blocksizes. */
typedef struct nf4_qweight {
  const uint8_t *packed;
  const float *absmax;
  const int8_t *absmax_q;
  const float *absmax_scale;
  int64_t n;
  int32_t blocksize;  /* power of two in [32, 4096] */
  int32_t quant_type; /* nf4_quant_type */
  int32_t double_quant;
  int32_t blocksize2; /* power of two in [64, 4096]; read when double_quant == 1 */
} nf4_qweight;

/* ------------------------------------------------------------ host helpers */

int32_t nf4_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *nf4_status_string(int32_t status);

/* ceil(n / 2) bytes of packed codes; -1 if n < 0. */
int64_t nf4_packed_bytes(int64_t n);

/* ceil(n / blocksize) blocks; -1 on n < 0 or blocksize <= 0. */
int64_t nf4_num_blocks(int64_t n, int32_t blocksize);

/* Writes the 16 fp32 code values, indexed by the 4-bit code, to the HOST array
 * `values`. NF4 [NF4 page, table 数学原理对比 row 数值表示]: quantiles of a
 * standard normal truncated at 929/960, 7 negative levels, an exact zero and 8
 * positive levels, scaled so the extremes are -1 and +1. FP4 [NF4 page, notes
 * 补充说明]: E2M1 values / 6. Derived on the host by the library itself. */
nf4_status nf4_codebook(int32_t quant_type, float values[16]);

/* Returns NF4_OK if the current HIP device can run the kernels (gfx950). */
nf4_status nf4_device_check(void);

/* ----------------------------------------------------------- compute calls */

/* Blockwise 4-bit quantization [NF4 page, table 数学原理对比 rows 缩放机制 and
 * 量化目标; repo page 0.49.2 blocksizes, 0.50.2 masked absmax store].
 * In:  w_bf16 [n] bf16, flattened.
 * Out: packed [ceil(n/2)], absmax [nb] (always written, also with double
 *      quant, where it is the intermediate), and when double_quant != 0 also
 *      absmax_q [nb] and absmax_scale [ceil(nb/256)] (blocksize2 = 256).
 * Per block: a = max|x|; s = RN(x / a) (s = 0 when a = 0); code = nearest
 * codebook value to s, an exact tie going to the smaller value; FP4 encodes
 * zero as nibble 0. absmax_q/absmax_scale may be NULL when double_quant == 0. */
nf4_status nf4_quantize(const void *w_bf16, int64_t n, int32_t blocksize, int32_t quant_type,
                        int32_t double_quant, uint8_t *packed, float *absmax, int8_t *absmax_q,
                        float *absmax_scale, void *stream);

/* Double quantization of block scales to 8 bits [NF4 page, table 实际性能差异
 * row 训练稳定性（QLoRA）]. Groups of blocksize2 consecutive absmax values; per
 * group m = max|a|, s2 = RN(m / 127) (0 when m = 0), q = clamp(rint(RN(a / s2)),
 * -127, 127) with ties to even. In: absmax [nb]. Out: absmax_q [nb],
 * absmax_scale [ceil(nb/blocksize2)]. */
nf4_status nf4_double_quant(const float *absmax, int64_t nb, int32_t blocksize2, int8_t *absmax_q,
                            float *absmax_scale, void *stream);

/* Dequantization [usage page, Configuration: compute dtype]. Out [w->n] as fp32
 * (out_dtype NF4_DTYPE_FP32: w = RN(c[code] * a')) or bf16 (NF4_DTYPE_BF16:
 * RNE_bf16 of that fp32 value), where a' = absmax, or RN(q * s2) with double
 * quant. */
nf4_status nf4_dequantize(const nf4_qweight *w, int32_t out_dtype, void *out, void *stream);

/* Largest `count` accepted by nf4_quantize_grouped and nf4_dequantize_grouped. */
#define NF4_QUANT_MAX_GROUP 16

/* Quantization of several tensors in one call -- e.g. the weights of one
 * transformer layer [NF4 page, table 数学原理对比; repo page 0.49.2]: for
 * i < count, exactly nf4_quantize(w_bf16[i], n[i], blocksize, quant_type,
 * double_quant, packed[i], absmax[i], absmax_q[i], absmax_scale[i]), with the
 * same argument rules per tensor. w_bf16, n, packed, absmax, absmax_q and
 * absmax_scale are HOST arrays of `count` entries (the buffers they point to are
 * on the device); absmax_q and absmax_scale may be NULL when double_quant == 0.
 * With double quantization at blocksize 64, 128 or 256 the tensors share one
 * launch, so small tensors do not each pay a launch's start-up and tail;
 * otherwise they are launched one after another. Every output is bitwise what
 * nf4_quantize writes for that tensor alone. 0 <= count <= NF4_QUANT_MAX_GROUP. */
nf4_status nf4_quantize_grouped(int32_t count, const void *const *w_bf16, const int64_t *n,
                                int32_t blocksize, int32_t quant_type, int32_t double_quant,
                                uint8_t *const *packed, float *const *absmax,
                                int8_t *const *absmax_q, float *const *absmax_scale,
                                void *stream);

/* Dequantization of several tensors in one launch [usage page, Configuration:
 * compute dtype]: for i < count, exactly nf4_dequantize(&w[i], out_dtype,
 * out[i]). w and out are HOST arrays of `count` entries; all tensors share the
 * quant type and the double-quant flag (NF4_ERR_UNSUPPORTED otherwise);
 * sizes and blocksizes may differ. Every output is bitwise what
 * nf4_dequantize writes for that tensor alone.
 * 0 <= count <= NF4_QUANT_MAX_GROUP. */
nf4_status nf4_dequantize_grouped(int32_t count, const nf4_qweight *w, int32_t out_dtype,
                                  void *const *out, void *stream);

/* Decode product for small batches [repo page 0.50.0: 4-bit GEMV and fused
 * 4-bit dequantize + GEMM for batch 1..64]:
 *   y[m, j] = sum_k bf16(dequant(W)[j, k]) * x[m, k],  fp32 accumulation,
 * x bf16 [M, K] row-major, W the quantized [N, K] tensor (w->n == N*K), y [M, N]
 * row-major in out_dtype (bf16 = RNE of the fp32 result). 1 <= M <= 16;
 * K <= 2^26 (NF4_ERR_UNSUPPORTED above).
 * compute_dtype must be NF4_DTYPE_BF16. The reduction order is fixed, so
 * repeated calls give identical bits. */
nf4_status nf4_gemv(const void *x_bf16, int32_t M, const nf4_qweight *w, int32_t N, int32_t K,
                    int32_t compute_dtype, int32_t out_dtype, void *y, void *stream);

/* Largest `count` accepted by nf4_gemv_grouped. */
#define NF4_GEMV_MAX_GROUP 16

/* Several independent decode products in ONE launch -- e.g. the projections of
 * one transformer layer at one decode position [repo page 0.50.0: kernels for
 * 4-bit inference chosen by shape; one launch keeps all CUs busy where a single
 * small GEMV cannot]. For i < count:
 *   y[i][m, j] = sum_k bf16(dequant(w[i])[j, k]) * x[i][m, k],
 * with the layouts and rules of nf4_gemv for each product. x_bf16, w, N, K and
 * y are HOST arrays of `count` entries (the tensors they point to are on the
 * device). All products share M (1..16), the quant type and the double-quant
 * flag (NF4_ERR_UNSUPPORTED otherwise); shapes and blocksizes may differ.
 * 0 <= count <= NF4_GEMV_MAX_GROUP. Each product's result is bitwise the same
 * as nf4_gemv on it alone. */
nf4_status nf4_gemv_grouped(int32_t count, const void *const *x_bf16, int32_t M,
                            const nf4_qweight *w, const int32_t *N, const int32_t *K,
                            int32_t compute_dtype, int32_t out_dtype, void *const *y,
                            void *stream);

/* Prefill product, any M >= 1: the same contraction as nf4_gemv, computed with
 * bf16 matrix cores on dequantized weight tiles and fp32 accumulation [repo
 * page 0.50.0: fused 4-bit dequantize + GEMM in place of dequantize +
 * F.linear]. Same layouts and rules as nf4_gemv, except that M is any
 * M >= 0, and K <= 2^22 and N <= 2^21 (NF4_ERR_UNSUPPORTED above). */
nf4_status nf4_gemm(const void *x_bf16, int32_t M, const nf4_qweight *w, int32_t N, int32_t K,
                    int32_t compute_dtype, int32_t out_dtype, void *y, void *stream);

/* Largest M that nf4_linear sends to the decode kernels (nf4_gemv's range). */
#define NF4_GEMV_MAX_M 16

/* A 4-bit linear layer with an optional fused bias, the kernel picked from the
 * shape [repo page ossradar.top bitsandbytes, release notes 0.50.0,
 * "Highlights": the new fused 4-bit kernels take the bias as well, and the
 * kernel is selected at run time from the shape]:
 *   y[m, j] = RN_fp32( sum_k bf16(dequant(W)[j, k]) * x[m, k] ) + bias[j]
 * with the sum accumulated in fp32 exactly as nf4_gemv / nf4_gemm do, then the
 * bf16 bias added in fp32, then the output rounding (bf16 = RNE of that fp32
 * value). bias_bf16: device [N] bf16, 2-byte aligned (NF4_ERR_MISALIGNED
 * otherwise), or NULL for none. 0 <= M <= NF4_GEMV_MAX_M runs nf4_gemv's
 * kernels, larger M nf4_gemm's, with their layouts, limits and errors. Without
 * a bias the result is bitwise that of nf4_gemv / nf4_gemm. */
nf4_status nf4_linear(const void *x_bf16, int32_t M, const nf4_qweight *w, int32_t N, int32_t K,
                      const void *bias_bf16, int32_t compute_dtype, int32_t out_dtype, void *y,
                      void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NF4_H */
