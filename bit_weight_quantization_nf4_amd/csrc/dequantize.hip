// dequantize.hip -- 4-bit codes back to fp32 or to the bf16 compute dtype.
//
// [usage page icman.com.cn/news/48546, "Configuration": the compute dtype is
//  the precision used after 4-bit dequantization, bf16 preferred; NF4 page,
//  table 数学原理对比, row 缩放机制: value = code value x block scale.]
// w = RN(c[code] * a'), a' = absmax or RN(q * s2); bf16 output = RNE(w).
//
// Layout: a wave owns tiles of 1024 consecutive elements and a lane owns
// elements 8l..8l+7 and 512+8l..512+8l+7 of each (one 4-byte code load per
// half; 8 | blocksize, so the 8 share one block scale). Each bf16 store
// instruction then writes 1 KB without gaps. Stores are non-temporal: the
// output is written once and not read back by this kernel, so it should not
// displace other lines from L2. The 16 fp32 code values sit in LDS; a code
// times 4 is cut from the packed word with one bit-field extract and used as
// the LDS byte offset.
#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kThreads = 256;

struct DequantArgs {
  const uint8_t *packed;
  void *out;
  int64_t n;
  ScaleArgs sc;
  int32_t log2_bs;
  float value[16];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(DequantArgs args) {
  __shared__ float table[16];
  if (threadIdx.x < 16) table[threadIdx.x] = args.value[threadIdx.x];
  __syncthreads();
  const char *tb = reinterpret_cast<const char *>(table);

  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t ntiles = (args.n + 1023) / 1024;
  for (int64_t tile = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6; tile < ntiles;
       tile += nwaves) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int64_t e0 = tile * 1024 + 512 * half + 8 * lane;
      if (e0 >= args.n) continue;
      const float ap = block_scale(args.sc, e0 >> args.log2_bs);
      const bool full = e0 + 8 <= args.n;
      uint32_t word;
      if (full) {
        word = *reinterpret_cast<const uint32_t *>(args.packed + e0 / 2);
      } else {
        const int64_t nbytes = (args.n - e0 + 1) / 2;
        word = 0;
        for (int i = 0; i < 4; ++i)
          if (i < nbytes) word |= (uint32_t)args.packed[e0 / 2 + i] << (8 * i);
      }
      // byte j of the word holds element 2j in bits 7..4 and 2j+1 in bits 3..0
      const uint32_t even4 = (word >> 2) & 0x3c3c3c3cu;  // 4 * code(2j) in byte j
      const uint32_t odd4 = (word << 2) & 0x3c3c3c3cu;   // 4 * code(2j+1) in byte j
      float w[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[2 * j] = *reinterpret_cast<const float *>(tb + ((even4 >> (8 * j)) & 0xffu)) * ap;
        w[2 * j + 1] = *reinterpret_cast<const float *>(tb + ((odd4 >> (8 * j)) & 0xffu)) * ap;
      }
      if (OUT_BF16) {
        uint16_t *o = reinterpret_cast<uint16_t *>(args.out) + e0;
        u32x4 v;
        v.x = pack_bf16x2(w[0], w[1]);
        v.y = pack_bf16x2(w[2], w[3]);
        v.z = pack_bf16x2(w[4], w[5]);
        v.w = pack_bf16x2(w[6], w[7]);
        if (full) {
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(o));
        } else {
          const uint32_t pk[4] = {v.x, v.y, v.z, v.w};
          for (int i = 0; i < 8 && e0 + i < args.n; ++i)
            o[i] = (uint16_t)(pk[i / 2] >> (16 * (i & 1)));
        }
      } else {
        float *o = reinterpret_cast<float *>(args.out) + e0;
        if (full) {
          f32x4 v0, v1;
          v0.x = w[0]; v0.y = w[1]; v0.z = w[2]; v0.w = w[3];
          v1.x = w[4]; v1.y = w[5]; v1.z = w[6]; v1.w = w[7];
          __builtin_nontemporal_store(v0, reinterpret_cast<f32x4 *>(o));
          __builtin_nontemporal_store(v1, reinterpret_cast<f32x4 *>(o) + 1);
        } else {
          for (int i = 0; i < 8 && e0 + i < args.n; ++i) o[i] = w[i];
        }
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
  args.sc = sc;
  args.log2_bs = __builtin_ctz((unsigned)blocksize);
  for (int i = 0; i < 16; ++i) args.value[i] = t.value[i];
  // one 1024-element tile per wave, at most 16 workgroups per CU
  int64_t blocks = ((n + 1023) / 1024 + kThreads / 64 - 1) / (kThreads / 64);
  if (blocks > 256 * 16) blocks = 256 * 16;
  dim3 grid((unsigned)blocks);
  if (out_bf16)
    hipLaunchKernelGGL(dequantize_kernel<true>, grid, dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL(dequantize_kernel<false>, grid, dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace nf4
