// double_quant.hip -- second-level quantization of the fp32 block scales.
//
// [NF4 page, CSDN "bitsandbytes 是一个用于高效量化和加载大型语言模型（LLM）的开源库",
//  table 实际性能差异, row 训练稳定性（QLoRA）: with use_double_quant the NF4
//  scales are quantized again with INT8 to shrink the metadata.]
// Per group of bs2 consecutive absmax values: m = max|a| (exact), s2 = RN(m/127)
// (0 for an all-zero group), q = clamp(rint(RN(a/s2)), -127, 127), ties to even.
// Divisions are the correctly rounded IEEE ones.
//
// The mean-centred variant (a reading; the page says only INT8) is below.
//
// Layout: a lane holds 4 consecutive values (16-byte load, one 32-bit store of
// four int8); G = min(64, bs2/4) lanes share a group and reduce its max across
// lanes; groups larger than 256 values loop R = bs2/256 times per lane.
#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int8_t q8(float a, float s2) {
  if (s2 == 0.0f) return 0;
  float r = __builtin_rintf(a / s2);
  r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
  return (int8_t)(int)r;
}

template <int BS2>
__global__ __launch_bounds__(kThreads) void double_quant_kernel(const float *__restrict__ absmax,
                                                                int64_t nb, int8_t *__restrict__ q,
                                                                float *__restrict__ s2out,
                                                                int64_t ntiles) {
  constexpr int G = BS2 / 4 < 64 ? BS2 / 4 : 64;  // lanes per group
  constexpr int R = BS2 / (4 * G);                 // 4-value chunks per lane
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  const int g = lane % G;

  for (int64_t tile = wave; tile < ntiles; tile += nwaves) {
    const int64_t group = tile * (64 / G) + lane / G;
    const int64_t base = group * BS2 + (int64_t)g * 4;
    float v[R][4];
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const int64_t e0 = base + (int64_t)c * G * 4;
      if (e0 + 4 <= nb) {
        float4 t = *reinterpret_cast<const float4 *>(absmax + e0);
        v[c][0] = t.x; v[c][1] = t.y; v[c][2] = t.z; v[c][3] = t.w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[c][j] = (e0 + j < nb) ? absmax[e0 + j] : 0.0f;
      }
    }
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < R; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(v[c][j]));
#pragma unroll
    for (int off = 1; off < G; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));

    const float s2 = (m == 0.0f) ? 0.0f : m / 127.0f;
    const int64_t ngroups = (nb + BS2 - 1) / BS2;
    if (g == 0 && group < ngroups) s2out[group] = s2;
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const int64_t e0 = base + (int64_t)c * G * 4;
      if (e0 >= nb) continue;
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) word |= ((uint32_t)(uint8_t)q8(v[c][j], s2)) << (8 * j);
      if (e0 + 4 <= nb) {
        *reinterpret_cast<uint32_t *>(q + e0) = word;
      } else {
        for (int j = 0; j < 4 && e0 + j < nb; ++j) q[e0 + j] = (int8_t)((word >> (8 * j)) & 0xff);
      }
    }
  }
}

// ---- the mean-centred second level -------------------------------------
// Per group of bs2 = 64 V scales, one wave: lane l holds values V l .. V l + V
// - 1 (zero past nb). The mean's sum is the pairwise one in index order: each
// lane adds its V values level by level (adjacent pairs first), then the
// lanes combine with xor-partners 1, 2, 4, ..., 32, which continues the same
// tree (fp32 addition is commutative, so both partners compute the same node).
// mu = RN(S / L) over the group's L real values; D = max |RN(a - mu)|;
// s2 = RN(D / 127) (0 if D = 0); q = clamp(rint(RN(RN(a - mu) / s2)), -127, 127).
template <int V>
__global__ __launch_bounds__(kThreads) void double_quant_centred_kernel(
    const float *__restrict__ absmax, int64_t nb, int8_t *__restrict__ q,
    float *__restrict__ s2out, float *__restrict__ muout, int64_t ngroups) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t group = wave; group < ngroups; group += nwaves) {
    const int64_t g0 = group * (64 * V);
    const int64_t e0 = g0 + (int64_t)lane * V;
    const int64_t L = nb - g0 < 64 * V ? nb - g0 : 64 * V;
    float v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = (e0 + j < nb) ? absmax[e0 + j] : 0.0f;
    float t[V];
#pragma unroll
    for (int j = 0; j < V; ++j) t[j] = v[j];
#pragma unroll
    for (int w = V; w > 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w / 2; ++i) t[i] = t[2 * i] + t[2 * i + 1];
    float S = t[0];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) S = S + __shfl_xor(S, off, 64);
    const float mu = S / (float)L;
    float D = 0.0f;
#pragma unroll
    for (int j = 0; j < V; ++j)
      if (e0 + j < nb) D = fmaxf(D, fabsf(v[j] - mu));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) D = fmaxf(D, __shfl_xor(D, off, 64));
    const float s2 = (D == 0.0f) ? 0.0f : D / 127.0f;
    if (lane == 0) {
      s2out[group] = s2;
      muout[group] = mu;
    }
#pragma unroll
    for (int j = 0; j < V; ++j)
      if (e0 + j < nb) q[e0 + j] = q8(v[j] - mu, s2);
  }
}

}  // namespace

hipError_t launch_double_quant_centred(const float *absmax, int64_t nb, int blocksize2, int8_t *q,
                                       float *s2, float *mu, hipStream_t stream) {
  if (nb == 0) return hipSuccess;
  const int64_t groups = (nb + blocksize2 - 1) / blocksize2;
  int64_t blocks = (groups + (kThreads / 64) - 1) / (kThreads / 64);
  if (blocks > 256 * 16) blocks = 256 * 16;
  dim3 grid((unsigned)blocks);
  switch (blocksize2) {
#define NF4_DQCCASE(V)                                                                       \
  case 64 * V:                                                                               \
    hipLaunchKernelGGL(double_quant_centred_kernel<V>, grid, dim3(kThreads), 0, stream, absmax, \
                       nb, q, s2, mu, groups);                                               \
    break;
    NF4_DQCCASE(1)
    NF4_DQCCASE(2)
    NF4_DQCCASE(4)
    NF4_DQCCASE(8)
    NF4_DQCCASE(16)
    NF4_DQCCASE(32)
    NF4_DQCCASE(64)
#undef NF4_DQCCASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_double_quant(const float *absmax, int64_t nb, int blocksize2, int8_t *q,
                               float *s2, hipStream_t stream) {
  if (nb == 0) return hipSuccess;
  const int G = blocksize2 / 4 < 64 ? blocksize2 / 4 : 64;
  const int64_t groups = (nb + blocksize2 - 1) / blocksize2;
  const int64_t per_tile = 64 / G;
  const int64_t ntiles = (groups + per_tile - 1) / per_tile;
  int64_t blocks = (ntiles + (kThreads / 64) - 1) / (kThreads / 64);
  if (blocks > 256 * 16) blocks = 256 * 16;
  dim3 grid((unsigned)blocks);
  switch (blocksize2) {
#define NF4_DQCASE(V)                                                                          \
  case V:                                                                                      \
    hipLaunchKernelGGL(double_quant_kernel<V>, grid, dim3(kThreads), 0, stream, absmax, nb, q, \
                       s2, ntiles);                                                            \
    break;
    NF4_DQCASE(64)
    NF4_DQCASE(128)
    NF4_DQCASE(256)
    NF4_DQCASE(512)
    NF4_DQCASE(1024)
    NF4_DQCASE(2048)
    NF4_DQCASE(4096)
#undef NF4_DQCASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nf4
