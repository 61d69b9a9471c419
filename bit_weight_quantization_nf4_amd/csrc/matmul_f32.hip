// matmul_f32.hip -- the products in the fp32 compute dtype:
//   y[m, n] = sum_k w[n, k] * x[m, k],  w = RN(c[code] * a') kept in fp32,
// fp32 activations, fp32 accumulation (one fused multiply-add per term), an
// optional fp32 bias added before the output rounding.
//
// [usage page icman.com.cn/news/48546, "Configuration": the compute dtype is
//  the precision used after 4-bit dequantization -- bf16 preferred, float32
//  and float16 the alternatives.]
//
// A straightforward tiled kernel on the fp32 vector units (the fp32 matrix
// cores have the same peak): a workgroup of 256 threads computes a BM x 64
// tile of y, walking K in steps of 32. Each step, every thread dequantizes one
// 8-code word of the weight tile into LDS (k-major, so neighbouring threads
// read neighbouring columns) and the x tile is staged beside it; each thread
// then accumulates BM / 16 x 4 outputs.
#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int BN = 64, BK = 32, kThreads = 256;

struct F32Args {
  const float *x;
  const uint8_t *packed;
  char *y;
  const float *bias;
  ScaleArgs sc;
  int32_t M, N, K;
  int64_t ldx, ldy;
  int32_t log2_bs;
  int32_t out_dtype;
  float value[16];
};

template <int BM, int DQ>
__global__ __launch_bounds__(kThreads) void matmul_f32_kernel(F32Args args) {
  constexpr int RM = BM / 16;  // output rows per thread
  __shared__ float table[16];
  __shared__ float xs[BK][BM + 1];
  __shared__ float ws[BK][BN + 1];
  if (threadIdx.x < 16) table[threadIdx.x] = args.value[threadIdx.x];
  const int tid = threadIdx.x;
  const int tm = tid / 16, tn = tid % 16;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = args.M, N = args.N, K = args.K;
  float acc[RM][4];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  // this thread's weight word: row n0 + tid / 4, codes 8 (tid % 4) .. + 7 of the step
  const int wr = tid / 4, wk = 8 * (tid % 4);
  const int wn = n0 + wr;
  __syncthreads();
  for (int k0 = 0; k0 < K; k0 += BK) {
    float w[8];
    if (wn < N) {
      const int64_t e = (int64_t)wn * K + k0 + wk;
      const uint32_t word = *reinterpret_cast<const uint32_t *>(args.packed + e / 2);
      const int64_t b = e >> args.log2_bs;
      float ap;
      if (DQ == kDqNone) {
        ap = args.sc.absmax[b];
      } else {
        const int64_t g = b >> args.sc.log2_bs2;
        ap = scale_from<DQ>(args.sc.absmax_q[b], args.sc.absmax_scale[g],
                            DQ == kDqCentred ? args.sc.absmax_offset[g] : 0.0f);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t byte = (word >> (8 * j)) & 0xffu;
        w[2 * j] = table[byte >> 4] * ap;
        w[2 * j + 1] = table[byte & 15] * ap;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) ws[wk + j][wr] = w[j];
    for (int i = tid; i < BM * BK; i += kThreads) {
      const int r = i / BK, kk = i % BK;
      const int m = m0 + r;
      xs[kk][r] = m < M ? args.x[(int64_t)m * args.ldx + k0 + kk] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < BK; ++kk) {
      float a[RM], bb[4];
#pragma unroll
      for (int i = 0; i < RM; ++i) a[i] = xs[kk][tm + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = ws[kk][tn + 16 * j];
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + tm + 16 * i, n = n0 + tn + 16 * j;
      if (m >= M || n >= N) continue;
      float v = acc[i][j];
      if (args.bias != nullptr) v += args.bias[n];
      const int64_t o = (int64_t)m * args.ldy + n;
      if (args.out_dtype == kFP32)
        reinterpret_cast<float *>(args.y)[o] = v;
      else if (args.out_dtype == kFP16)
        reinterpret_cast<uint16_t *>(args.y)[o] = (uint16_t)out_bits<kFP16>(v);
      else
        reinterpret_cast<uint16_t *>(args.y)[o] = (uint16_t)out_bits<kBF16>(v);
    }
}

template <int BM>
void launch_bm(const F32Args &args, dim3 grid, int dq, hipStream_t stream) {
  if (dq == kDqCentred)
    hipLaunchKernelGGL((matmul_f32_kernel<BM, kDqCentred>), grid, dim3(kThreads), 0, stream, args);
  else if (dq == kDqSym)
    hipLaunchKernelGGL((matmul_f32_kernel<BM, kDqSym>), grid, dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((matmul_f32_kernel<BM, kDqNone>), grid, dim3(kThreads), 0, stream, args);
}

}  // namespace

hipError_t launch_matmul_f32(const GemvDesc &d, int M, int quant_type, int out_dtype,
                             hipStream_t stream) {
  if (M == 0 || d.N == 0) return hipSuccess;
  const CodeTables &t = code_tables(quant_type);
  F32Args args;
  args.x = static_cast<const float *>(d.x);
  args.packed = d.packed;
  args.y = static_cast<char *>(d.y);
  args.bias = static_cast<const float *>(d.bias);
  args.sc = d.sc;
  args.M = M;
  args.N = d.N;
  args.K = d.K;
  args.ldx = d.ldx;
  args.ldy = d.ldy;
  args.log2_bs = __builtin_ctz((unsigned)d.blocksize);
  args.out_dtype = out_dtype;
  for (int i = 0; i < 16; ++i) args.value[i] = t.value[i];
  const int bm = M <= 16 ? 16 : 64;
  const dim3 grid((unsigned)((d.N + BN - 1) / BN), (unsigned)((M + bm - 1) / bm));
  if (grid.y > 65535) return hipErrorInvalidValue;
  if (bm == 16) launch_bm<16>(args, grid, d.sc.double_quant, stream);
  else launch_bm<64>(args, grid, d.sc.double_quant, stream);
  return hipGetLastError();
}

}  // namespace nf4
