// gemm.hip -- prefill product Y[M, N] = X[M, K] . bf16(dequant(W))[N, K]^T on
// gfx950 bf16 matrix cores, fp32 accumulation.
//
// [repo page ossradar.top bitsandbytes, release notes 0.50.0: a fused 4-bit
//  dequantize + GEMM replaces dequantize + F.linear; usage page
//  icman.com.cn/news/48546, "Configuration": bf16 compute dtype after 4-bit
//  dequantization.]
//
// Tiling: a workgroup of 4 waves computes a BM x BN = 128 x 128 tile of Y and
// walks K in steps of BK = 64. Per step it stages the X tile (bf16) and the
// weight tile -- read as packed codes and dequantized on the fly to the same
// bf16 values the dequantize kernel produces -- in LDS, then each wave runs
// 2 x 2 v_mfma_f32_32x32x16_bf16 tiles (64 x 64 outputs) over the four
// 16-wide k-steps. LDS rows are padded by 16 bytes so the 16-byte operand
// reads of 8 consecutive lanes cover all banks once.
#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kLdsStride = BK + 8;  // bf16 elements per LDS row

struct GemmArgs {
  const uint16_t *x;
  const uint8_t *packed;
  void *y;
  int32_t M, N, K;
  int32_t log2_bs;
  ScaleArgs sc;
  float value[16];
};

__device__ __forceinline__ uint4 dequant8_u4(uint32_t word, float ap, const char *tb) {
  const uint32_t even4 = (word >> 2) & 0x3c3c3c3cu;
  const uint32_t odd4 = (word << 2) & 0x3c3c3c3cu;
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float c0 = *reinterpret_cast<const float *>(tb + ((even4 >> (8 * j)) & 0xffu));
    const float c1 = *reinterpret_cast<const float *>(tb + ((odd4 >> (8 * j)) & 0xffu));
    out[j] = pack_bf16x2(c0 * ap, c1 * ap);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[BM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t ws[BN * kLdsStride];
  __shared__ float table[16];
  if (threadIdx.x < 16) table[threadIdx.x] = args.value[threadIdx.x];
  __syncthreads();
  const char *tb = reinterpret_cast<const char *>(table);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = args.M, N = args.N, K = args.K;

  // staging assignment: thread -> (row, 32-wide half of the BK slice)
  const int srow = tid >> 1, shalf = tid & 1;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += BK) {
    const int kk = k0 + 32 * shalf;  // K % 32 == 0: a 32-wide piece is all in or all out
    // X tile piece: 32 bf16 of row m0 + srow
    uint4 xv[4];
    {
      const int m = m0 + srow;
      const bool ok = m < M && kk < K;
      const uint16_t *src = args.x + (int64_t)m * K + kk;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xv[i] = ok ? reinterpret_cast<const uint4 *>(src)[i] : make_uint4(0, 0, 0, 0);
    }
    // W tile piece: 32 codes of row n0 + srow, dequantized to bf16
    uint4 wv[4];
    {
      const int n = n0 + srow;
      if (n < N && kk < K) {
        const int64_t e = (int64_t)n * K + kk;
        const uint4 p = *reinterpret_cast<const uint4 *>(args.packed + e / 2);
        const float ap = block_scale(args.sc, e >> args.log2_bs);
        wv[0] = dequant8_u4(p.x, ap, tb);
        wv[1] = dequant8_u4(p.y, ap, tb);
        wv[2] = dequant8_u4(p.z, ap, tb);
        wv[3] = dequant8_u4(p.w, ap, tb);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[i] = make_uint4(0, 0, 0, 0);
      }
    }
    __syncthreads();  // previous step's operand reads are done
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4 *>(&xs[srow * kLdsStride + 32 * shalf + 8 * i]) = xv[i];
      *reinterpret_cast<uint4 *>(&ws[srow * kLdsStride + 32 * shalf + 8 * i]) = wv[i];
    }
    __syncthreads();

#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      // 32x32x16 operands: lane l holds row (l % 32), k = 8 * (l / 32) .. +7
      const int kcol = ks * 16 + 8 * (lane >> 5);
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + 32 * i + (lane & 31);
        a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(&xs[r * kLdsStride + kcol]));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + 32 * j + (lane & 31);
        b[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(&ws[r * kLdsStride + kcol]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // D layout of the 32x32 MFMA: lane l holds column l % 32 and, for register
  // r, row 8 * (r / 4) + 4 * (l / 32) + r % 4.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int n = n0 + wn * 64 + 32 * j + (lane & 31);
        if (m < M && n < N) {
          const int64_t o = (int64_t)m * N + n;
          if (OUT_BF16)
            reinterpret_cast<uint16_t *>(args.y)[o] =
                (uint16_t)(pack_bf16x2(acc[i][j][r], 0.0f) & 0xffffu);
          else
            reinterpret_cast<float *>(args.y)[o] = acc[i][j][r];
        }
      }
}

}  // namespace

hipError_t launch_gemm(const uint16_t *x, int M, const uint8_t *packed, int N, int K,
                       int blocksize, int quant_type, const ScaleArgs &sc, bool out_bf16,
                       void *y, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const CodeTables &t = code_tables(quant_type);
  GemmArgs args;
  args.x = x;
  args.packed = packed;
  args.y = y;
  args.M = M;
  args.N = N;
  args.K = K;
  args.log2_bs = __builtin_ctz((unsigned)blocksize);
  args.sc = sc;
  for (int i = 0; i < 16; ++i) args.value[i] = t.value[i];
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  if (out_bf16)
    hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace nf4
