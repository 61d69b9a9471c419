// nf4_internal.h -- host-side interface between the C ABI layer (nf4_api.hip)
// and the kernel launchers. Launchers assume validated arguments.
#pragma once

#include "nf4.h"
#include "nf4_common.h"

namespace nf4 {

// Tables for NF4 / FP4, derived on first use (nf4_tables.hip).
const CodeTables &code_tables(int quant_type);

hipError_t launch_quantize(const uint16_t *w, int64_t n, int blocksize, int quant_type,
                           uint8_t *packed, float *absmax, hipStream_t stream);

hipError_t launch_double_quant(const float *absmax, int64_t nb, int blocksize2, int8_t *q,
                               float *s2, hipStream_t stream);

// The mean-centred second level (offsets mu per group of blocksize2 scales).
hipError_t launch_double_quant_centred(const float *absmax, int64_t nb, int blocksize2, int8_t *q,
                                       float *s2, float *mu, hipStream_t stream);

// Quantization of a [rows, cols] matrix of bf16 / fp16 / fp32 elements whose
// rows start ld elements apart (any blocksize), as the flattened row-major
// tensor; absmax only (double quantization is a second launch). The code
// decisions use the correctly rounded quotient, so a contiguous bf16 input
// gives bitwise the codes of launch_quantize.
hipError_t launch_quantize_generic(const void *w, int w_dtype, int64_t rows, int64_t cols,
                                   int64_t ld, int blocksize, int quant_type, uint8_t *packed,
                                   float *absmax, hipStream_t stream);

// One tensor of a quantization launch (absmax_q / absmax_scale used with
// double quantization only).
struct QuantTensorDesc {
  const uint16_t *w;
  int64_t n;
  uint8_t *packed;
  float *absmax;
  int8_t *absmax_q;
  float *absmax_scale;
};

// Quantization and double quantization (groups of blocksize2 scales) in one
// launch, for the pairs where quantize_dq_fused() is true, over up to
// quantize_max_group() tensors that share blocksize and quant type; each
// tensor's results equal launch_quantize followed by launch_double_quant.
bool quantize_dq_fused(int blocksize, int blocksize2);
int quantize_max_group();
hipError_t launch_quantize_dq(int count, const QuantTensorDesc *ts, int blocksize, int quant_type,
                              hipStream_t stream);

// One tensor of a dequantization launch.
struct DequantDesc {
  const uint8_t *packed;
  int64_t n;
  int blocksize;
  ScaleArgs sc;
  void *out;
};

// Dequantization of up to dequantize_max_group() tensors in one launch; they
// share the quant type, the double-quant mode and the output dtype (kBF16,
// kFP16 or kFP32). Each tensor's output equals what it gets launched alone.
int dequantize_max_group();
hipError_t launch_dequantize(int count, const DequantDesc *ds, int quant_type, int dq,
                             int out_dtype, hipStream_t stream);

// One decode product of a group launched together by launch_gemv_grouped.
struct GemvDesc {
  const void *x;          // [M, K] in the compute dtype, row m at m * ldx elements
  const uint8_t *packed;  // [N*K/2]
  void *y;                // [M, N] in the output dtype, row m at m * ldy elements
  ScaleArgs sc;
  int32_t N, K, blocksize;
  const void *bias;       // [N] in the compute dtype, added in fp32 before the output rounding; or null
  int64_t ldx, ldy;
};

// Largest number of products in one grouped launch.
int gemv_max_group();

// Decode products (1 <= M <= 64) on the matrix cores. All products share M,
// K, the compute dtype (bf16 / fp16), the output dtype, the quant type (one
// code table) and the double-quant mode; blocksizes and N may differ (one
// blocksize per call takes the register-resident kernel). A product's result
// depends only on its own data, M, K and whether the call splits K: a
// product whose activations do not fit the registers of a CU
// (gemv_split_ranges(M, K) > 1) is split into K ranges when `workspace`
// holds the sum of gemv_split_bytes over the call's products (fp32 partial
// sums, 256-byte aligned per product); otherwise it streams x.
hipError_t launch_gemv_mt(int count, const GemvDesc *descs, int M, int K, int quant_type, int dq,
                          int compute_dtype, int out_dtype, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

// The summing launch of a K split: product i's S[i] fp32 partial-sum planes
// part[i][r][M][N_i] are added in range order, the bias (compute dtype) added,
// and the result rounded to the output dtype into descs[i].y (row stride ldy).
hipError_t launch_gemv_split_sum(int count, const GemvDesc *descs, float *const *part,
                                 const int *S, int M, int compute_dtype, int out_dtype,
                                 hipStream_t stream);

// The tiled decode kernel for 9 <= M <= 64 (x staged in LDS, K split over
// workgroups into gemv_tk_ranges(M, N, K) ranges, chosen from the product's
// shape and the CU count; 0 where the kernel does not apply). With more than
// one range a product needs gemv_tk_bytes(M, N, K) workspace bytes (256-byte
// aligned, the call's products consecutive in its order). A product's result
// depends only on its own data, its shape and the device's CU count.
// gemv_tk_enabled() is false when NF4_DECODE_TILED=0 is set in the
// environment (the register-resident kernel then takes these products).
int gemv_tk_ranges(int M, int N, int K);
size_t gemv_tk_bytes(int M, int N, int K);
bool gemv_tk_enabled();
hipError_t launch_gemv_tk(int count, const GemvDesc *descs, int M, int K, int quant_type, int dq,
                          int compute_dtype, int out_dtype, void *workspace, hipStream_t stream);

// 16-row MFMA tiles that hold M activation rows (1, 2 or 4).
int gemv_row_tiles(int M);
// K ranges a product of this M and K is split into (1: none; 0: more than
// the kernel takes, so it streams x).
int gemv_split_ranges(int M, int K);
// Workspace bytes of one such product's partial sums (0 without a split).
size_t gemv_split_bytes(int M, int N, int K);

// Single-activation-row products (M = 1) for K <= gemv1_max_k(blocksize): waves own
// whole rows; same grouping rules (contiguous x and y).
int gemv1_max_k(int blocksize);
hipError_t launch_gemv1_grouped(int count, const GemvDesc *descs, int quant_type,
                                bool double_quant, bool out_bf16, hipStream_t stream);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// NF4_LOG set (and not "0") in the environment: log_msg writes one line per
// dispatch decision to stderr, prefixed "[nf4] ". log_on() reads the variable
// once per process.
bool log_on();
void log_msg(const char *fmt, ...) __attribute__((format(printf, 1, 2)));

// Prefill GEMM, any M, compute dtype bf16 or fp16 (x, bias), output dtype
// kBF16 / kFP16 / kFP32; x rows ldx elements apart, y rows ldy apart.
// bias: [N] in the compute dtype, added in fp32 before the output rounding,
// or null.
hipError_t launch_gemm(const void *x, int64_t ldx, int M, const uint8_t *packed, int N, int K,
                       int blocksize, int quant_type, const ScaleArgs &sc, int compute_dtype,
                       int out_dtype, void *y, int64_t ldy, const void *bias, hipStream_t stream);

// The same GEMM with the weights already dequantized: w16 [N, K] in the
// compute dtype, rows ldw elements apart (the tile streams into LDS like x).
// With w16 = the dequantize kernel's output of a weight, its result is bitwise
// launch_gemm's on that weight.
hipError_t launch_gemm_w16(const void *x, int64_t ldx, int M, const void *w16, int64_t ldw, int N,
                           int K, int compute_dtype, int out_dtype, void *y, int64_t ldy,
                           const void *bias, hipStream_t stream);

// Products in the fp32 compute dtype (weights RN(c a') kept in fp32, fp32
// activations and bias, fp32 accumulation), any M; same descriptor rules.
hipError_t launch_matmul_f32(const GemvDesc &d, int M, int quant_type, int out_dtype,
                             hipStream_t stream);

// nf4_linear_ws and nf4_linear_workspace_bytes (the ABI layer), for the
// allocation-free entry point.
nf4_status linear_with_workspace(const void *x, int64_t ldx, int32_t M, const nf4_qweight *w,
                                 int32_t N, int32_t K, const void *bias, int32_t compute_dtype,
                                 int32_t out_dtype, void *y, int64_t ldy, void *workspace,
                                 int64_t workspace_bytes, void *stream);
int64_t linear_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t blocksize,
                               int32_t compute_dtype, int32_t out_dtype, int32_t double_quant);

}  // namespace nf4
