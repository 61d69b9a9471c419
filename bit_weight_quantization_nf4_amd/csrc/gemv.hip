// gemv.hip -- decode product y[M, N] = x[M, K] . bf16(dequant(W))[N, K]^T for
// 1 <= M <= 16, on gfx950 matrix cores.
//
// [repo page ossradar.top bitsandbytes, release notes 0.50.0: 4-bit inference
//  at batch 1 uses a 4-bit GEMV, batches 2..64 a fused 4-bit dequantize + GEMM
//  in place of dequantize + F.linear; usage page icman.com.cn/news/48546,
//  "Configuration": weights are dequantized to the bf16 compute dtype before
//  the product.]
//
// Design (memory-bound: the 4-bit weights are read once, x is tiny):
//  - one workgroup = 8 waves over 16*NG weight rows; the waves split K and
//    their partial sums are added in a fixed order through LDS, so results are
//    bitwise reproducible without atomics;
//  - the contraction runs on v_mfma_f32_16x16x32_bf16 with x as the A operand
//    (rows m >= M are zero) and the dequantized weights as the B operand.
//    Lane (n, kg) of the B operand needs 8 consecutive k of weight row n,
//    i.e. exactly one 32-bit word of packed codes; each lane loads 16 bytes =
//    32 codes (k-range 32kg..32kg+31 of a 128-wide chunk) and feeds four MFMAs.
//    The A operand is permuted the same way, so the k order inside the chunk
//    does not matter;
//  - dequantization per code: one bit-field extract of 4*code from a pre-shifted
//    word, one LDS read of the fp32 code value, one multiply by the block scale,
//    and half a v_cvt_pk_bf16_f32 -- exactly the dequantize kernel's bf16
//    weight, so the product is that of the bf16 compute-dtype weights.
#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 128;  // codes of one row per wave step

struct GemvArgs {
  const uint16_t *x;
  const uint8_t *packed;
  void *y;
  int32_t M, N, K;
  int32_t log2_bs;
  ScaleArgs sc;
  float value[16];
};

// 8 codes of one packed word -> 4 registers of bf16 pairs in k order.
__device__ __forceinline__ bf16x8 dequant8(uint32_t word, float ap, const char *tb) {
  const uint32_t even4 = (word >> 2) & 0x3c3c3c3cu;
  const uint32_t odd4 = (word << 2) & 0x3c3c3c3cu;
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float c0 = *reinterpret_cast<const float *>(tb + ((even4 >> (8 * j)) & 0xffu));
    const float c1 = *reinterpret_cast<const float *>(tb + ((odd4 >> (8 * j)) & 0xffu));
    out[j] = pack_bf16x2(c0 * ap, c1 * ap);
  }
  uint4 v = make_uint4(out[0], out[1], out[2], out[3]);
  return __builtin_bit_cast(bf16x8, v);
}

template <int NG, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs args) {
  __shared__ float table[16];
  __shared__ float red[kWaves][NG][4][64];
  if (threadIdx.x < 16) table[threadIdx.x] = args.value[threadIdx.x];
  __syncthreads();
  const char *tb = reinterpret_cast<const char *>(table);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;  // B column (weight row in the group) / A row (m)
  const int kg = lane >> 4;  // which 32-code piece of the chunk
  const int row0 = blockIdx.x * 16 * NG;
  const int K = args.K;
  const int nch = (K + kChunk - 1) / kChunk;
  const int c_begin = (wave * nch) / kWaves;
  const int c_end = ((wave + 1) * nch) / kWaves;

  f32x4 acc[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool m_ok = nl < args.M;
  const uint16_t *xrow = args.x + (int64_t)(m_ok ? nl : 0) * K;

  for (int c = c_begin; c < c_end; ++c) {
    const int k0 = c * kChunk + 32 * kg;
    const bool k_ok = k0 < K;  // K % 32 == 0: the piece is all in or all out
    uint4 xa[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      xa[s] = (m_ok && k_ok) ? *reinterpret_cast<const uint4 *>(xrow + k0 + 8 * s)
                             : make_uint4(0, 0, 0, 0);
    uint4 pw[NG];
    float ap[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int row = row0 + 16 * g + nl;
      if (row < args.N && k_ok) {
        const int64_t e = (int64_t)row * K + k0;
        pw[g] = *reinterpret_cast<const uint4 *>(args.packed + e / 2);
        ap[g] = block_scale(args.sc, e >> args.log2_bs);
      } else {
        pw[g] = make_uint4(0, 0, 0, 0);
        ap[g] = 0.0f;
      }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const uint32_t words[4] = {pw[g].x, pw[g].y, pw[g].z, pw[g].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 b = dequant8(words[s], ap[g], tb);
        bf16x8 a = __builtin_bit_cast(bf16x8, xa[s]);
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[g], 0, 0, 0);
      }
    }
  }

  // Cross-wave reduction in a fixed order.
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][g][r][lane] = acc[g][r];
  __syncthreads();
  for (int v = threadIdx.x; v < NG * 4 * 64; v += kThreads) {
    const int g = v / 256, r = (v / 64) % 4, l = v % 64;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += red[w][g][r][l];
    // D layout of the 16x16 MFMA: lane l holds rows 4*(l/16)+r of column l%16.
    const int m = 4 * (l >> 4) + r;
    const int n = row0 + 16 * g + (l & 15);
    if (m < args.M && n < args.N) {
      const int64_t o = (int64_t)m * args.N + n;
      if (OUT_BF16)
        reinterpret_cast<uint16_t *>(args.y)[o] = (uint16_t)(pack_bf16x2(sum, 0.0f) & 0xffffu);
      else
        reinterpret_cast<float *>(args.y)[o] = sum;
    }
  }
}

template <int NG>
hipError_t launch_ng(const GemvArgs &args, bool out_bf16, hipStream_t stream) {
  dim3 grid((unsigned)((args.N + 16 * NG - 1) / (16 * NG)));
  if (out_bf16)
    hipLaunchKernelGGL((gemv_kernel<NG, true>), grid, dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((gemv_kernel<NG, false>), grid, dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const uint16_t *x, int M, const uint8_t *packed, int N, int K,
                       int blocksize, int quant_type, const ScaleArgs &sc, bool out_bf16,
                       void *y, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const CodeTables &t = code_tables(quant_type);
  GemvArgs args;
  args.x = x;
  args.packed = packed;
  args.y = y;
  args.M = M;
  args.N = N;
  args.K = K;
  args.log2_bs = __builtin_ctz((unsigned)blocksize);
  args.sc = sc;
  for (int i = 0; i < 16; ++i) args.value[i] = t.value[i];
  // Wider row groups share each x chunk across more weight rows; keep at
  // least ~2 workgroups per CU.
  if (M > 4 && N >= 16 * 2 * 512) return launch_ng<2>(args, out_bf16, stream);
  return launch_ng<1>(args, out_bf16, stream);
}

}  // namespace nf4
