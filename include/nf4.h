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
 *  - Every device pointer must be 16-byte aligned (NF4_ERR_MISALIGNED);
 *    row strides of inputs (the *_ex calls) must keep every row 16-byte
 *    aligned.
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
 *    absmax_q int8[nb] and absmax_scale float[ceil(nb/blocksize2)], plus
 *    absmax_offset float[ceil(nb/blocksize2)] in the mean-centred mode;
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

#define NF4_ABI_VERSION 3

/* Largest M of the decode products (nf4_gemv, nf4_gemv_grouped); nf4_linear
 * sends M up to this to the decode kernels and larger M to the GEMM. */
#define NF4_GEMV_MAX_M 64

typedef enum nf4_status {
  NF4_OK = 0,
  NF4_ERR_INVALID_ARGUMENT = 1, /* NULL pointer, negative size, bad enum, shape mismatch */
  NF4_ERR_UNSUPPORTED = 2,      /* valid request this library does not implement, or not gfx950 */
  NF4_ERR_MISALIGNED = 3,       /* a device pointer is not 16-byte aligned */
  NF4_ERR_DEVICE = 4,           /* no HIP device, or a HIP call / launch failed */
  NF4_ERR_SCRATCH = 5           /* more workspace than nf4_linear_noalloc's static scratch */
} nf4_status;

typedef enum nf4_quant_type { NF4_QUANT_NF4 = 0, NF4_QUANT_FP4 = 1 } nf4_quant_type;

/* Element types of activations, outputs, biases and quantize inputs. The
 * compute dtype of a product is the type the 4-bit weights are dequantized to
 * before the multiply [usage page, "Configuration": bf16 preferred; fp16 and
 * fp32 also used; NF4 page, notes 补充说明: NF4 + double quant + FP16 compute]. */
typedef enum nf4_dtype { NF4_DTYPE_BF16 = 0, NF4_DTYPE_FP32 = 1, NF4_DTYPE_FP16 = 2 } nf4_dtype;

/* Second-level (double) quantization of the block scales [NF4 page, table
 * 实际性能差异 row 训练稳定性（QLoRA）: the NF4 scales are quantized again to
 * INT8]. Per group of blocksize2 consecutive absmax values:
 *  NF4_DQ_SYMMETRIC: m = max a, s2 = RN(m / 127) (0 if m = 0),
 *                    q = clamp(rint(RN(a / s2)), -127, 127); a' = RN(q s2).
 *  NF4_DQ_CENTRED:   mu = RN(S / L) with S the pairwise fp32 sum of the
 *                    group's L values zero-padded to blocksize2 (adjacent
 *                    pairs first, level by level), D = max |RN(a - mu)|,
 *                    s2 = RN(D / 127) (0 if D = 0),
 *                    q = clamp(rint(RN(RN(a - mu) / s2)), -127, 127);
 *                    a' = RN(RN(q s2) + mu). The codes use both signs. */
typedef enum nf4_double_quant_mode {
  NF4_DQ_NONE = 0,
  NF4_DQ_SYMMETRIC = 1,
  NF4_DQ_CENTRED = 2
} nf4_double_quant_mode;

/* Descriptor of one quantized tensor. The pointers are device pointers owned by
 * the caller; `absmax` is read when double_quant == NF4_DQ_NONE, `absmax_q`
 * and `absmax_scale` in both double-quant modes, `absmax_offset` in
 * NF4_DQ_CENTRED only; fields a mode does not read are ignored. Mirrors the
 * pages' configuration fields (quant_type, use_double_quant) plus the
 * blocksizes. */
typedef struct nf4_qweight {
  const uint8_t *packed;
  const float *absmax;
  const int8_t *absmax_q;
  const float *absmax_scale;
  int64_t n;
  int32_t blocksize;    /* power of two in [32, 4096] */
  int32_t quant_type;   /* nf4_quant_type */
  int32_t double_quant; /* nf4_double_quant_mode */
  int32_t blocksize2;   /* power of two in [64, 4096]; read with double quant */
  const float *absmax_offset; /* [ceil(nb / blocksize2)], NF4_DQ_CENTRED */
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
 * zero as nibble 0. absmax_q/absmax_scale may be NULL when double_quant == 0.
 * double_quant is NF4_DQ_NONE or NF4_DQ_SYMMETRIC here (nf4_quantize_ex takes
 * every mode, input type and row stride). */
nf4_status nf4_quantize(const void *w_bf16, int64_t n, int32_t blocksize, int32_t quant_type,
                        int32_t double_quant, uint8_t *packed, float *absmax, int8_t *absmax_q,
                        float *absmax_scale, void *stream);

/* The general form of nf4_quantize [NF4 page, table 数学原理对比; repo page
 * 0.49.2 release notes: quantize/dequantize accept non-contiguous tensors].
 * In:  w, a [rows, cols] matrix of w_dtype elements (NF4_DTYPE_BF16, FP16 or
 *      FP32) whose row r starts ld elements after row r - 1 (ld >= cols);
 *      it is quantized as the flattened row-major tensor of n = rows * cols
 *      elements, each element taken at its exact fp32 value. A strided
 *      matrix (ld > cols, rows > 1) needs cols % 8 == 0 (NF4_ERR_UNSUPPORTED
 *      otherwise) and 16-byte aligned rows.
 * Out: as nf4_quantize; double_quant is any nf4_double_quant_mode with
 *      blocksize2 = 256, and absmax_offset [ceil(nb/256)] is written in
 *      NF4_DQ_CENTRED (it may be NULL otherwise). For a contiguous bf16
 *      input and double_quant 0 or 1 the result is bitwise nf4_quantize's. */
nf4_status nf4_quantize_ex(const void *w, int32_t w_dtype, int64_t rows, int64_t cols, int64_t ld,
                           int32_t blocksize, int32_t quant_type, int32_t double_quant,
                           uint8_t *packed, float *absmax, int8_t *absmax_q, float *absmax_scale,
                           float *absmax_offset, void *stream);

/* Double quantization of block scales to 8 bits [NF4 page, table 实际性能差异
 * row 训练稳定性（QLoRA）]. Groups of blocksize2 consecutive absmax values; per
 * group m = max|a|, s2 = RN(m / 127) (0 when m = 0), q = clamp(rint(RN(a / s2)),
 * -127, 127) with ties to even. In: absmax [nb]. Out: absmax_q [nb],
 * absmax_scale [ceil(nb/blocksize2)]. */
nf4_status nf4_double_quant(const float *absmax, int64_t nb, int32_t blocksize2, int8_t *absmax_q,
                            float *absmax_scale, void *stream);

/* Double quantization in either mode (nf4_double_quant_mode; see its
 * comment for the arithmetic). In: absmax [nb]. Out: absmax_q [nb],
 * absmax_scale [ceil(nb/blocksize2)], and for NF4_DQ_CENTRED absmax_offset
 * [ceil(nb/blocksize2)] (may be NULL in NF4_DQ_SYMMETRIC, where the call is
 * nf4_double_quant). mode NF4_DQ_NONE is NF4_ERR_INVALID_ARGUMENT. */
nf4_status nf4_double_quant_ex(const float *absmax, int64_t nb, int32_t blocksize2, int32_t mode,
                               int8_t *absmax_q, float *absmax_scale, float *absmax_offset,
                               void *stream);

/* Dequantization [usage page, Configuration: compute dtype]. Out [w->n] as fp32
 * (out_dtype NF4_DTYPE_FP32: w = RN(c[code] * a')), bf16 (NF4_DTYPE_BF16:
 * RNE_bf16 of that fp32 value) or fp16 (NF4_DTYPE_FP16: RNE_fp16 of it), where
 * a' is the block's effective scale (absmax, or the double-quant a' of the
 * descriptor's mode). */
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
 *   y[m, j] = sum_k cd(dequant(W)[j, k]) * x[m, k],  fp32 accumulation,
 * with cd the rounding to compute_dtype (bf16 or fp16 RNE; none for fp32).
 * x [M, K] row-major in compute_dtype, W the quantized [N, K] tensor (w->n ==
 * N*K), y [M, N] row-major in out_dtype (bf16 / fp16 = RNE of the fp32
 * result). 1 <= M <= NF4_GEMV_MAX_M; K <= 2^26 (NF4_ERR_UNSUPPORTED above).
 * The reduction order is fixed, so repeated calls give identical bits. */
nf4_status nf4_gemv(const void *x, int32_t M, const nf4_qweight *w, int32_t N, int32_t K,
                    int32_t compute_dtype, int32_t out_dtype, void *y, void *stream);

/* Largest `count` accepted by nf4_gemv_grouped. */
#define NF4_GEMV_MAX_GROUP 16

/* Several independent decode products in ONE launch -- e.g. the projections of
 * one transformer layer at one decode position [repo page 0.50.0: kernels for
 * 4-bit inference chosen by shape; one launch keeps all CUs busy where a single
 * small GEMV cannot]. For i < count:
 *   y[i][m, j] = sum_k cd(dequant(w[i])[j, k]) * x[i][m, k],
 * with the layouts and rules of nf4_gemv for each product. x, w, N, K and y
 * are HOST arrays of `count` entries (the tensors they point to are on the
 * device). All products share M (1..NF4_GEMV_MAX_M), the compute dtype, the
 * quant type and the double-quant mode (NF4_ERR_UNSUPPORTED otherwise); shapes
 * and blocksizes may differ.
 * 0 <= count <= NF4_GEMV_MAX_GROUP. Each product's result is bitwise the same
 * as nf4_gemv on it alone. */
nf4_status nf4_gemv_grouped(int32_t count, const void *const *x, int32_t M,
                            const nf4_qweight *w, const int32_t *N, const int32_t *K,
                            int32_t compute_dtype, int32_t out_dtype, void *const *y,
                            void *stream);

/* Prefill product, any M >= 0: the same contraction as nf4_gemv, computed with
 * matrix cores (bf16 / fp16 compute) on dequantized weight tiles and fp32
 * accumulation [repo page 0.50.0: fused 4-bit dequantize + GEMM in place of
 * dequantize + F.linear]. Same layouts and rules as nf4_gemv, except that M
 * is any M >= 0, and K <= 2^22 and N <= 2^21 (NF4_ERR_UNSUPPORTED above). */
nf4_status nf4_gemm(const void *x, int32_t M, const nf4_qweight *w, int32_t N, int32_t K,
                    int32_t compute_dtype, int32_t out_dtype, void *y, void *stream);


/* A 4-bit linear layer with an optional fused bias, the kernel picked from the
 * shape [repo page ossradar.top bitsandbytes, release notes 0.50.0,
 * "Highlights": the new fused 4-bit kernels take the bias as well, and the
 * kernel is selected at run time from the shape]:
 *   y[m, j] = RN_fp32( sum_k cd(dequant(W)[j, k]) * x[m, k] ) + bias[j]
 * with the sum accumulated in fp32 exactly as nf4_gemv / nf4_gemm do, then the
 * bias (compute_dtype, widened exactly) added in fp32, then the output
 * rounding (bf16 / fp16 = RNE of that fp32 value). bias: device [N] in
 * compute_dtype, aligned to its element size (NF4_ERR_MISALIGNED otherwise),
 * or NULL for none. 0 <= M <= NF4_GEMV_MAX_M runs nf4_gemv's kernels, larger
 * M nf4_gemm's, with their layouts, limits and errors. Without a bias the
 * result is bitwise that of nf4_gemv / nf4_gemm. */
nf4_status nf4_linear(const void *x, int32_t M, const nf4_qweight *w, int32_t N, int32_t K,
                      const void *bias, int32_t compute_dtype, int32_t out_dtype, void *y,
                      void *stream);

/* nf4_linear on strided activations and outputs [repo page, release notes
 * 0.49.2: non-contiguous tensors are accepted]: row m of x starts ldx
 * elements after row m - 1 (ldx >= K) and row m of y ldy elements after row
 * m - 1 (ldy >= N); every row of x must start 16-byte aligned
 * (NF4_ERR_MISALIGNED otherwise; y needs only its element alignment). With ldx == K and ldy == N it is
 * nf4_linear; otherwise the result equals nf4_linear on contiguous copies,
 * bit for bit, and elements of y outside the [M, N] window are not written. */
nf4_status nf4_linear_ex(const void *x, int64_t ldx, int32_t M, const nf4_qweight *w, int32_t N,
                         int32_t K, const void *bias, int32_t compute_dtype, int32_t out_dtype,
                         void *y, int64_t ldy, void *stream);

/* Prefill products (bf16 / fp16 compute) of at least this many rows take the
 * dequantized-weight path of nf4_linear_ws when the workspace allows. */
#define NF4_PREFILL_DEQUANT_MIN_M 1536

/* Bytes of device workspace nf4_linear_ws uses for one product of this shape
 * and these types (double_quant is the nf4_double_quant_mode; blocksize as in
 * nf4_qweight), 0 when its kernels need none. For a prefill product of at
 * least NF4_PREFILL_DEQUANT_MIN_M rows (bf16 / fp16 compute) it is 2 * N * K,
 * rounded up to 256: room for W dequantized once to the compute dtype, which
 * the GEMM then reads instead of dequantizing each weight tile again for every
 * 256-row tile of x [usage page icman.com.cn/news/48546, "Configuration":
 * 4-bit weights are dequantized to the compute dtype for the matmul]. Among
 * decode shapes (M <= NF4_GEMV_MAX_M, bf16 / fp16 compute) it is non-zero for
 * those whose activations, x[M,
 * K], do not fit the registers of one compute unit -- 8 <= M <= 16 with K >
 * 6144, 17 <= M <= 32 with K > 4096, M > 32 with K > 2048 (at most 8 K ranges;
 * fewer rows, or longer K, stream x) -- which are then split along K: each K
 * range is summed into fp32 partials in the workspace and a second kernel adds
 * the ranges in order. Where that split would take two (M <= 16) or three
 * (M > 16) or more ranges and K <= 16384 (at 8 rows, every such product), a
 * tiled kernel takes the product
 * with a split of its own (up to 8 ranges of at most 2048 codes, as many as
 * keep the product within one round of workgroups on the device's compute
 * units), so the size depends on N and the CU count as well [repo page
 * ossradar.top bitsandbytes, release notes
 * 0.50.0, "Highlights": fused 4-bit kernels for batch 2..64, chosen at run
 * time from the shape]. At most S * M * N * 4 bytes (S <= 8 K ranges),
 * rounded up to 256. Never negative. */
int64_t nf4_linear_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t blocksize,
                                   int32_t compute_dtype, int32_t out_dtype,
                                   int32_t double_quant);

/* nf4_linear_ex with a caller-owned device workspace (16-byte aligned;
 * workspace_bytes >= 0, and workspace non-NULL when workspace_bytes > 0,
 * else NF4_ERR_INVALID_ARGUMENT / NF4_ERR_MISALIGNED). With workspace_bytes >=
 * nf4_linear_workspace_bytes(M, N, K, w->blocksize, compute_dtype, out_dtype,
 * w->double_quant) a decode product that the query sizes is split along K as
 * described there, and a prefill product it sizes dequantizes W into the
 * workspace and runs the GEMM on it (the same tiles, MFMA order and weight
 * values as the fused GEMM, so bitwise nf4_linear_ex's result); with less (or
 * none) the call is nf4_linear_ex, bit for bit. The split changes the
 * summation order, not the accuracy contract: the
 * result is within the same fp32 bounds, and repeated calls with a workspace
 * give identical bits. The workspace holds no state between calls; it must
 * not be used by other work on the device while the call runs (calls on one
 * stream may share one workspace). */
nf4_status nf4_linear_ws(const void *x, int64_t ldx, int32_t M, const nf4_qweight *w, int32_t N,
                         int32_t K, const void *bias, int32_t compute_dtype, int32_t out_dtype,
                         void *y, int64_t ldy, void *workspace, int64_t workspace_bytes,
                         void *stream);

/* nf4_gemv_grouped with a caller-owned device workspace, as for nf4_linear_ws:
 * with workspace_bytes at least the sum over the products of
 * nf4_linear_workspace_bytes, every product that query sizes is split along K;
 * each product's result is bitwise that of nf4_linear_ws on it alone with a
 * sufficient workspace (no bias, contiguous x and y). */
nf4_status nf4_gemv_grouped_ws(int32_t count, const void *const *x, int32_t M,
                               const nf4_qweight *w, const int32_t *N, const int32_t *K,
                               int32_t compute_dtype, int32_t out_dtype, void *const *y,
                               void *workspace, int64_t workspace_bytes, void *stream);

/* Size of the static scratch nf4_linear_noalloc uses (one per device). */
#define NF4_NOALLOC_SCRATCH_BYTES (32u << 20)

/* For callers that cannot allocate device memory -- code under stream capture,
 * tight serving loops, harnesses that forbid allocation: nf4_linear_ws with
 * the workspace taken from a static device array of NF4_NOALLOC_SCRATCH_BYTES
 * (32 MiB) that the library holds on each device it runs on until the process
 * ends; nothing is allocated or freed by the call. Same arguments, layouts,
 * results (bitwise those of nf4_linear_ws with a sufficient workspace) and
 * errors as nf4_linear_ex, plus NF4_ERR_SCRATCH, returned before anything is
 * launched, when a decode product's nf4_linear_workspace_bytes exceeds
 * NF4_NOALLOC_SCRATCH_BYTES. Prefill products (M > NF4_GEMV_MAX_M) take the
 * fused GEMM and no scratch. The scratch holds only partial sums that each
 * call writes before reading, so it needs no clearing; but every call on one
 * device shares it, so calls that may overlap on one device (other streams,
 * other host threads) race and must be serialised by the caller. */
nf4_status nf4_linear_noalloc(const void *x, int64_t ldx, int32_t M, const nf4_qweight *w,
                              int32_t N, int32_t K, const void *bias, int32_t compute_dtype,
                              int32_t out_dtype, void *y, int64_t ldy, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NF4_H */
