// dequantize.hip -- 4-bit codes back to fp32 or to the bf16 compute dtype.
//
// [usage page icman.com.cn/news/48546, "Configuration": the compute dtype is
//  the precision used after 4-bit dequantization, bf16 preferred; NF4 page,
//  table 数学原理对比, row 缩放机制: value = code value x block scale.]
// w = RN(c[code] * a'), a' = absmax or RN(q * s2); bf16 output = RNE(w).
//
// Layout: a lane owns 16 consecutive codes (one 8-byte load; 16 | blocksize so
// they share one block scale) and writes 32 B (bf16) or 64 B (fp32) with
// 16-byte stores. The 16 fp32 code values sit in LDS; a code times 4 is cut
// from the packed word with one bit-field extract and used as the LDS byte
// offset.
#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kThreads = 256;

struct DequantArgs {
  const uint8_t *packed;
  void *out;
  int64_t n;
  int64_t nchunks;  // ceil(n / 16)
  ScaleArgs sc;
  int32_t log2_bs;
  float value[16];
};

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(DequantArgs args) {
  __shared__ float table[16];
  if (threadIdx.x < 16) table[threadIdx.x] = args.value[threadIdx.x];
  __syncthreads();
  const char *tb = reinterpret_cast<const char *>(table);

  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t chunk = (int64_t)blockIdx.x * kThreads + threadIdx.x; chunk < args.nchunks;
       chunk += stride) {
    const int64_t e0 = chunk * 16;
    const float ap = block_scale(args.sc, e0 >> args.log2_bs);
    const bool full = e0 + 16 <= args.n;
    uint2 p;
    if (full) {
      p = *reinterpret_cast<const uint2 *>(args.packed + e0 / 2);
    } else {
      uint32_t b[8];
      const int64_t nbytes = (args.n - e0 + 1) / 2;
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = (i < nbytes) ? args.packed[e0 / 2 + i] : 0u;
      p.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
      p.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    }
    float w[16];
    const uint32_t words[2] = {p.x, p.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // byte j of the word holds element 2j in bits 7..4 and 2j+1 in bits 3..0
      const uint32_t even4 = (words[h] >> 2) & 0x3c3c3c3cu;  // 4 * code(2j) in byte j
      const uint32_t odd4 = (words[h] << 2) & 0x3c3c3c3cu;   // 4 * code(2j+1) in byte j
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float c0 = *reinterpret_cast<const float *>(tb + ((even4 >> (8 * j)) & 0xffu));
        const float c1 = *reinterpret_cast<const float *>(tb + ((odd4 >> (8 * j)) & 0xffu));
        w[8 * h + 2 * j] = c0 * ap;
        w[8 * h + 2 * j + 1] = c1 * ap;
      }
    }
    if (OUT_BF16) {
      uint16_t *o = reinterpret_cast<uint16_t *>(args.out) + e0;
      uint32_t pk[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pk[i] = pack_bf16x2(w[2 * i], w[2 * i + 1]);
      if (full) {
        reinterpret_cast<uint4 *>(o)[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        reinterpret_cast<uint4 *>(o)[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
      } else {
        for (int i = 0; i < 16 && e0 + i < args.n; ++i)
          o[i] = (uint16_t)(pk[i / 2] >> (16 * (i & 1)));
      }
    } else {
      float *o = reinterpret_cast<float *>(args.out) + e0;
      if (full) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          reinterpret_cast<float4 *>(o)[i] =
              make_float4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
      } else {
        for (int i = 0; i < 16 && e0 + i < args.n; ++i) o[i] = w[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_dequantize(const uint8_t *packed, int64_t n, int blocksize, int quant_type,
                             const ScaleArgs &sc, bool out_bf16, void *out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const CodeTables &t = code_tables(quant_type);
  DequantArgs args;
  args.packed = packed;
  args.out = out;
  args.n = n;
  args.nchunks = (n + 15) / 16;
  args.sc = sc;
  args.log2_bs = __builtin_ctz((unsigned)blocksize);
  for (int i = 0; i < 16; ++i) args.value[i] = t.value[i];
  int64_t blocks = (args.nchunks + kThreads - 1) / kThreads;
  if (blocks > 256 * 16) blocks = 256 * 16;
  dim3 grid((unsigned)blocks);
  if (out_bf16)
    hipLaunchKernelGGL(dequantize_kernel<true>, grid, dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL(dequantize_kernel<false>, grid, dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace nf4
