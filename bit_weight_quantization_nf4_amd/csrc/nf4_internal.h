// nf4_internal.h -- host-side interface between the C ABI layer (nf4_api.hip)
// and the kernel launchers. Launchers assume validated arguments.
#pragma once

#include "nf4_common.h"

namespace nf4 {

// Tables for NF4 / FP4, derived on first use (nf4_tables.hip).
const CodeTables &code_tables(int quant_type);

hipError_t launch_quantize(const uint16_t *w, int64_t n, int blocksize, int quant_type,
                           uint8_t *packed, float *absmax, hipStream_t stream);

hipError_t launch_double_quant(const float *absmax, int64_t nb, int blocksize2, int8_t *q,
                               float *s2, hipStream_t stream);

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
// share the quant type, the double-quant flag and the output dtype. Each
// tensor's output equals what it gets launched alone.
int dequantize_max_group();
hipError_t launch_dequantize(int count, const DequantDesc *ds, int quant_type, bool double_quant,
                             bool out_bf16, hipStream_t stream);

// One decode product of a group launched together by launch_gemv_grouped.
struct GemvDesc {
  const uint16_t *x;      // [M, K] bf16
  const uint8_t *packed;  // [N*K/2]
  void *y;                // [M, N]
  ScaleArgs sc;
  int32_t N, K, blocksize;
  const uint16_t *bias;   // [N] bf16, added in fp32 before the output rounding; or null
};

// Largest number of products in one grouped launch.
int gemv_max_group();

// All products share M, the quant type (one code table) and the double-quant
// flag; blocksizes and shapes may differ.
hipError_t launch_gemv_grouped(int count, const GemvDesc *descs, int M, int quant_type,
                               bool double_quant, bool out_bf16, hipStream_t stream);

// Single-activation-row products (M = 1) for K <= gemv1_max_k(): waves own
// whole rows; same grouping rules as launch_gemv_grouped.
int gemv1_max_k();
hipError_t launch_gemv1_grouped(int count, const GemvDesc *descs, int quant_type,
                                bool double_quant, bool out_bf16, hipStream_t stream);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// bias: [N] bf16 added in fp32 before the output rounding, or null
hipError_t launch_gemm(const uint16_t *x, int M, const uint8_t *packed, int N, int K,
                       int blocksize, int quant_type, const ScaleArgs &sc, bool out_bf16,
                       void *y, const uint16_t *bias, hipStream_t stream);

}  // namespace nf4
