// quantize.hip -- blockwise NF4/FP4 quantization on gfx950.
//
// [NF4 page, CSDN "bitsandbytes 是一个用于高效量化和加载大型语言模型（LLM）的开源库",
//  table 数学原理对比, rows 缩放机制 (each block gets its own scale max|x|,
//  values normalised into [-1, 1]) and 量化目标 (nearest code value);
//  repo page ossradar.top bitsandbytes, release notes 0.49.2 (1-D blocksize 64
//  default, 32/128 also used; bs 64 on wave64 CDNA) and 0.50.2 (mask the absmax
//  store of the partial last block).]
//
// Layout of the work: a lane owns E = max(8, bs/64) elements of one block,
// read as 16-byte vectors; G = bs/E lanes share a block and reduce its absmax
// with cross-lane max. Each 8-element chunk becomes one 32-bit word of packed
// nibbles, so loads and stores are fully coalesced.
//
// Per element: s = x / a; the code is read from a 33-cell lookup indexed by
// RN(16 s + 16) (one fma gives that integer exactly), which holds the one
// decision threshold that can fall inside the cell and the codes on either
// side of it. Division: q0 = x * RN(1/a) gives the same NF4 code as the
// correctly rounded RN(x/a) for every bf16 (x, a) pair (checked exhaustively
// over all significand/exponent classes); FP4 adds the residual correction
// q1 = q0 + (x - q0 a) RN(1/a) with two fmas, which equals RN(x/a) wherever
// the result is normal. Both hold while 1/a, the product and the residual stay
// normal, i.e. for a in [2^-100, 2^120); other blocks take a true division.
#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kThreads = 256;

struct QuantArgs {
  const uint16_t *w;
  uint8_t *packed;
  float *absmax;
  int64_t n;
  int64_t nb;
  int64_t ntiles;
  float cell_thr[kCells];
  uint32_t cell_codes[kCells];
};

template <int QT>
__device__ __forceinline__ float normalise(float x, float a, float r, bool fast) {
  if (fast) {
    float q0 = x * r;
    if (QT == kQuantNF4) return q0;
    float e = __builtin_fmaf(-q0, a, x);
    return __builtin_fmaf(e, r, q0);
  }
  return x / a;
}

// Code of one normalised value through the LDS cell lookup. Finite inputs give
// cells 0..32; the mask keeps a NaN (from non-finite input) inside the table.
constexpr int kLutSize = 64;

__device__ __forceinline__ uint32_t code_of(float s, const uint2 *lut) {
  float t = __builtin_fmaf(s, 16.0f, 8388624.0f);  // 2^23 + 16 + 16 s, rounded to an integer
  uint32_t cell = (__float_as_uint(t) - 0x4B000000u) & (kLutSize - 1);
  uint2 e = lut[cell];
  return (s > __uint_as_float(e.x)) ? (e.y >> 16) : (e.y & 0xffffu);
}

template <int QT>
__device__ __forceinline__ uint32_t encode8(const uint32_t d[4], float a, float r, bool fast,
                                            const uint2 *lut) {
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // d[j] holds elements 2j (low half) and 2j+1 (high half): byte j of the
    // output is code(2j) << 4 | code(2j+1).
    float x0 = __uint_as_float(d[j] << 16);
    float x1 = __uint_as_float(d[j] & 0xffff0000u);
    uint32_t c0 = code_of(normalise<QT>(x0, a, r, fast), lut);
    uint32_t c1 = code_of(normalise<QT>(x1, a, r, fast), lut);
    word |= (c0 << (8 * j + 4)) | (c1 << (8 * j));
  }
  return word;
}

__device__ __forceinline__ uint32_t absmax_bits16(const uint32_t d[4]) {
  u16x2 m = __builtin_bit_cast(u16x2, d[0] & 0x7fff7fffu);
#pragma unroll
  for (int j = 1; j < 4; ++j)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, d[j] & 0x7fff7fffu));
  return m.x > m.y ? m.x : m.y;
}

template <int BS, int QT>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs args) {
  constexpr int E = BS / 64 > 8 ? BS / 64 : 8;  // elements per lane per block
  constexpr int G = BS / E;                      // lanes per block (<= 64)
  constexpr int CH = E / 8;                      // 8-element chunks per lane

  __shared__ uint2 lut[kLutSize];
  if (threadIdx.x < kLutSize) {
    const int c = threadIdx.x < kCells ? threadIdx.x : kCells - 1;
    lut[threadIdx.x] = make_uint2(__float_as_uint(args.cell_thr[c]), args.cell_codes[c]);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  const int g = lane % G;  // position inside the block's lane group

  for (int64_t tile = wave; tile < args.ntiles; tile += nwaves) {
    const int64_t block = tile * (64 / G) + lane / G;
    const int64_t base = block * BS + (int64_t)g * 8;  // first element of chunk 0
    uint32_t d[CH][4];
    bool full[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t e0 = base + (int64_t)c * G * 8;
      full[c] = e0 + 8 <= args.n;
      if (full[c]) {
        uint4 v = *reinterpret_cast<const uint4 *>(args.w + e0);
        d[c][0] = v.x; d[c][1] = v.y; d[c][2] = v.z; d[c][3] = v.w;
      } else {
        // ragged tail: elements at or past n read as +0
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t lo = (e0 + 2 * j < args.n) ? args.w[e0 + 2 * j] : 0u;
          uint32_t hi = (e0 + 2 * j + 1 < args.n) ? args.w[e0 + 2 * j + 1] : 0u;
          d[c][j] = lo | (hi << 16);
        }
      }
    }

    // block absmax: exact max of |x| in bf16 bit space, then across the group
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      uint32_t mc = absmax_bits16(d[c]);
      m = m > mc ? m : mc;
    }
#pragma unroll
    for (int off = 1; off < G; off <<= 1) {
      uint32_t o = __shfl_xor(m, off, 64);
      m = m > o ? m : o;
    }
    const float a = bf16_bits_to_f32(m);
    if (g == 0 && block < args.nb) args.absmax[block] = a;

    const bool fast = (a == 0.0f) || (a >= 0x1p-100f && a < 0x1p120f);
    const float r = (a == 0.0f) ? 0.0f : 1.0f / a;

#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t e0 = base + (int64_t)c * G * 8;
      if (e0 >= args.n) continue;
      uint32_t word = encode8<QT>(d[c], a, r, fast, lut);
      if (full[c]) {
        *reinterpret_cast<uint32_t *>(args.packed + e0 / 2) = word;
      } else {
        // ragged tail: clear the nibbles of missing elements, store only the
        // bytes that exist (ceil(n/2) in total)
        const int64_t valid = args.n - e0;  // 1..7
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (2 * b >= valid) break;
          uint32_t byte = (word >> (8 * b)) & 0xffu;
          if (2 * b + 1 >= valid) byte &= 0xf0u;
          args.packed[e0 / 2 + b] = (uint8_t)byte;
        }
      }
    }
  }
}

template <int QT>
hipError_t launch_qt(int blocksize, dim3 grid, QuantArgs args, hipStream_t stream) {
  switch (blocksize) {
#define NF4_QCASE(BSV)                                                                   \
  case BSV:                                                                              \
    hipLaunchKernelGGL((quantize_kernel<BSV, QT>), grid, dim3(kThreads), 0, stream, args); \
    break;
    NF4_QCASE(32)
    NF4_QCASE(64)
    NF4_QCASE(128)
    NF4_QCASE(256)
    NF4_QCASE(512)
    NF4_QCASE(1024)
    NF4_QCASE(2048)
    NF4_QCASE(4096)
#undef NF4_QCASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const uint16_t *w, int64_t n, int blocksize, int quant_type,
                           uint8_t *packed, float *absmax, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const CodeTables &t = code_tables(quant_type);
  QuantArgs args;
  args.w = w;
  args.packed = packed;
  args.absmax = absmax;
  args.n = n;
  args.nb = (n + blocksize - 1) / blocksize;
  const int E = blocksize / 64 > 8 ? blocksize / 64 : 8;
  const int64_t tile_elems = 64LL * E;
  args.ntiles = (n + tile_elems - 1) / tile_elems;
  for (int i = 0; i < kCells; ++i) {
    args.cell_thr[i] = t.cell_thr[i];
    args.cell_codes[i] = t.cell_codes[i];
  }
  // Enough waves to keep every CU's memory pipeline busy; each wave then
  // strides over the remaining tiles.
  const int64_t waves_wanted = args.ntiles;
  int64_t blocks = (waves_wanted + (kThreads / 64) - 1) / (kThreads / 64);
  const int64_t max_blocks = 256 * 16;
  if (blocks > max_blocks) blocks = max_blocks;
  dim3 grid((unsigned)blocks);
  return quant_type == kQuantFP4 ? launch_qt<kQuantFP4>(blocksize, grid, args, stream)
                                 : launch_qt<kQuantNF4>(blocksize, grid, args, stream);
}

}  // namespace nf4
