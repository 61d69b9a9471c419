// quantize.hip -- blockwise NF4/FP4 quantization on gfx950.
//
// [NF4 page, CSDN "bitsandbytes 是一个用于高效量化和加载大型语言模型（LLM）的开源库",
//  table 数学原理对比, rows 缩放机制 (each block gets its own scale max|x|,
//  values normalised into [-1, 1]) and 量化目标 (nearest code value);
//  repo page ossradar.top bitsandbytes, release notes 0.49.2 (1-D blocksize 64
//  default, 32/128 also used; bs 64 on wave64 CDNA) and 0.50.2 (mask the absmax
//  store of the partial last block).]
//
// Layout of the work: a wave takes tiles of 64 * E elements, E = max(32,
// bs/64); each 512-element chunk of a tile is one contiguous 16-byte load per
// lane (8 elements) and one 4-byte store of their packed nibbles. The lanes of
// a block reduce its absmax with cross-lane max. A wave keeps the loads of its
// next tile in flight while it encodes the current one. With double
// quantization at bs 64/128/256 one launch also quantizes the scales: a
// workgroup owns each group of 256 blocks and meets its scales in LDS.
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

// Elements per lane of one tile: E = max(32, bs / 64), in E / 8 chunks of 8.
// Chunk c of a tile is its elements [512 c, 512 c + 512): lane l owns
// 512 c + 8 l .. +7, so every 16-byte load and 4-byte store instruction covers
// one contiguous range. A block of bs <= 512 elements is G = bs / 8 lanes of
// one chunk; a larger block is bs / 512 whole chunks.
template <int BS>
constexpr int lane_elems() { return BS / 64 > 32 ? BS / 64 : 32; }

template <int BS>
struct TileShape {
  static constexpr int E = lane_elems<BS>();
  static constexpr int CH = E / 8;      // chunks per lane (per tile)
  static constexpr int kTile = 64 * E;  // elements per tile
};

// Loads of one tile through a buffer resource whose range is the tile's bytes
// rounded up to whole 16-byte granules (w is 16-byte aligned and so is every
// tile, so the range never leaves the granule of element n - 1, and a
// granule never crosses a page): granules past the end read as 0 without a
// branch. In the last, ragged tile the elements at or past n inside the final
// granule are then cleared explicitly.
template <int BS>
__device__ __forceinline__ void load_tile(uint32_t (&d)[TileShape<BS>::CH][4],
                                          const QuantArgs &args, int64_t tile, int lane) {
  constexpr int CH = TileShape<BS>::CH, kTile = TileShape<BS>::kTile;
  const int64_t t0 = tile * kTile;
  const int64_t rem = args.n - t0;
  const int64_t valid = rem < kTile ? (rem > 0 ? rem : 0) : kTile;
  const uint32_t bytes = (uint32_t)((2 * valid + 15) & ~(int64_t)15);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(args.w + (t0 < args.n ? t0 : 0)), (short)0, (int)bytes, 0x00020000);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const uint4 v = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(1024 * c + 16 * lane), 0, 0));
    d[c][0] = v.x; d[c][1] = v.y; d[c][2] = v.z; d[c][3] = v.w;
  }
  if (valid < kTile) {
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t e = 512 * c + 8 * lane + 2 * j;  // element of the low half
        if (e >= valid) d[c][j] = 0u;
        else if (e + 1 >= valid) d[c][j] &= 0xffffu;
      }
  }
}

// Absmax, codes and stores of one tile; mb[c] returns the bf16 bits of the
// absmax of chunk c's block (every lane of the block holds it).
template <int BS, int QT, bool kStoreAbsmax = true>
__device__ __forceinline__ void encode_tile(const uint32_t (&d)[TileShape<BS>::CH][4],
                                            const QuantArgs &args, int64_t tile, int lane,
                                            const uint2 *lut,
                                            uint32_t (&mb)[TileShape<BS>::CH]) {
  constexpr int CH = TileShape<BS>::CH, kTile = TileShape<BS>::kTile;
  const int64_t t0 = tile * kTile;
  // scale of each chunk: the absmax of its block, exact, in bf16 bit space
  if constexpr (BS <= 512) {
    constexpr int G = BS / 8;  // lanes per block
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      uint32_t m = absmax_bits16(d[c]);
#pragma unroll
      for (int off = 1; off < G; off <<= 1) {
        const uint32_t o = __shfl_xor(m, off, 64);
        m = m > o ? m : o;
      }
      mb[c] = m;
      const int64_t block = (t0 + 512 * c + 8 * lane) / BS;
      if (kStoreAbsmax && lane % G == 0 && block < args.nb) args.absmax[block] = bf16_bits_to_f32(m);
    }
  } else {
    constexpr int CPB = BS / 512;  // chunks per block
#pragma unroll
    for (int j = 0; j < CH / CPB; ++j) {
      uint32_t m = 0;
#pragma unroll
      for (int c = j * CPB; c < (j + 1) * CPB; ++c) {
        const uint32_t mc = absmax_bits16(d[c]);
        m = m > mc ? m : mc;
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_xor(m, off, 64);
        m = m > o ? m : o;
      }
#pragma unroll
      for (int c = j * CPB; c < (j + 1) * CPB; ++c) mb[c] = m;
      const int64_t block = t0 / BS + j;
      if (kStoreAbsmax && lane == 0 && block < args.nb) args.absmax[block] = bf16_bits_to_f32(m);
    }
  }

  const bool whole_tile = t0 + kTile <= args.n;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const float a = bf16_bits_to_f32(mb[c]);
    const bool fast = (a == 0.0f) || (a >= 0x1p-100f && a < 0x1p120f);
    const float r = (a == 0.0f) ? 0.0f : 1.0f / a;
    const uint32_t word = encode8<QT>(d[c], a, r, fast, lut);
    const int64_t e0 = t0 + 512 * c + 8 * lane;
    if (whole_tile) {
      *reinterpret_cast<uint32_t *>(args.packed + e0 / 2) = word;
    } else if (e0 < args.n) {
      // ragged tail: clear the nibbles of missing elements, store only the
      // bytes that exist (ceil(n/2) in total)
      const int64_t valid = args.n - e0;
      if (valid >= 8) {
        *reinterpret_cast<uint32_t *>(args.packed + e0 / 2) = word;
      } else {
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

__device__ __forceinline__ void load_lut(uint2 *lut, const QuantArgs &args) {
  if (threadIdx.x < kLutSize) {
    const int c = threadIdx.x < kCells ? threadIdx.x : kCells - 1;
    lut[threadIdx.x] = make_uint2(__float_as_uint(args.cell_thr[c]), args.cell_codes[c]);
  }
  __syncthreads();
}

template <int BS, int QT>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs args) {
  constexpr int CH = TileShape<BS>::CH;
  __shared__ uint2 lut[kLutSize];
  load_lut(lut, args);

  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);

  // two tiles in flight per wave: the loads of the next tile are issued
  // before the current one is encoded
  uint32_t da[CH][4], db[CH][4], mb[CH];
  int64_t tile = wave;
  if (tile < args.ntiles) load_tile<BS>(da, args, tile, lane);
  for (; tile < args.ntiles; tile += 2 * nwaves) {
    const int64_t t1 = tile + nwaves;
    load_tile<BS>(db, args, t1 < args.ntiles ? t1 : tile, lane);
    encode_tile<BS, QT>(da, args, tile, lane, lut, mb);
    if (t1 >= args.ntiles) break;
    const int64_t t2 = t1 + nwaves;
    load_tile<BS>(da, args, t2 < args.ntiles ? t2 : t1, lane);
    encode_tile<BS, QT>(db, args, t1, lane, lut, mb);
  }
}

// Quantization with the double quantization of its block scales in the same
// pass [NF4 page, CSDN "bitsandbytes 是一个用于高效量化和加载大型语言模型（LLM）的开源库",
// table 实际性能差异, row 训练稳定性（QLoRA）: the block scales are quantized
// again with INT8]. A workgroup owns one group of 256 blocks at a time, TPW
// tiles per wave; the scales of the group meet in LDS, where every wave takes
// their maximum, and the threads then store the fp32 absmax and the int8 code
// of one block each, so both stores are coalesced. The arithmetic is that of
// the separate double-quant kernel: m = fmaxf over the group, s2 = RN(m / 127)
// (0 for m = 0), q = clamp(rint(RN(a / s2)), -127, 127), ties to even.
__device__ __forceinline__ int8_t dq_code(float a, float s2) {
  if (s2 == 0.0f) return 0;
  float r = __builtin_rintf(a / s2);
  r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
  return (int8_t)(int)r;
}

constexpr int kGroupBlocks = 256;
constexpr int64_t kMaxDqGroups = 256 * 8;  // workgroups of one fused launch

// W waves per group: 4 in general (three workgroups fit a CU), 8 when there
// are too few groups to give every CU more than one workgroup.
template <int BS, int W>
struct DqShape {
  static constexpr int TPG = kGroupBlocks * BS / TileShape<BS>::kTile;  // tiles per group
  static constexpr int TPW = TPG / W;                                   // tiles per wave
  static constexpr int kThreads = 64 * W;
};

template <int BS, int QT, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(3))) void quantize_dq_kernel(
    QuantArgs args, int8_t *absmax_q, float *absmax_scale, int64_t ngroups) {
  constexpr int CH = TileShape<BS>::CH, kTile = TileShape<BS>::kTile;
  constexpr int TPG = DqShape<BS, W>::TPG, TPW = DqShape<BS, W>::TPW, NT = DqShape<BS, W>::kThreads;
  static_assert(BS <= 512 && TPW % 2 == 0 && TPG % TPW == 0, "an even number of tiles per wave");
  constexpr int G = BS / 8;  // lanes per block within a chunk

  __shared__ uint2 lut[kLutSize];
  __shared__ float sabs[2][kGroupBlocks];
  if (threadIdx.x < kLutSize) {
    const int c = threadIdx.x < kCells ? threadIdx.x : kCells - 1;
    lut[threadIdx.x] = make_uint2(__float_as_uint(args.cell_thr[c]), args.cell_codes[c]);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t first_tile = (int64_t)wave * TPW;

  uint32_t buf[2][CH][4], mb[CH];
  int64_t group = blockIdx.x;
  if (group < ngroups) load_tile<BS>(buf[0], args, group * TPG + first_tile, lane);
  for (int it = 0; group < ngroups; group += gridDim.x, ++it) {
    float *sa = sabs[it & 1];
    // tiles in pairs, so that the register buffer of each is known at compile time
#pragma unroll 1
    for (int tp = 0; tp < TPW; tp += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = tp + u;
        const int64_t tile = group * TPG + first_tile + t;
        // the last tile of the group prefetches the first of the next group
        const int64_t next = t + 1 < TPW ? tile + 1
                             : (group + gridDim.x < ngroups ? (group + gridDim.x) * TPG + first_tile
                                                            : tile);
        load_tile<BS>(buf[u ^ 1], args, next, lane);
        encode_tile<BS, QT, false>(buf[u], args, tile, lane, lut, mb);
#pragma unroll
        for (int c = 0; c < CH; ++c)
          if (lane % G == 0)
            sa[((first_tile + t) * kTile + 512 * c + 8 * lane) / BS] = bf16_bits_to_f32(mb[c]);
      }
    }
    __syncthreads();
    // group maximum (blocks past n hold 0), taken by every wave
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < kGroupBlocks / 64; ++k) m = fmaxf(m, sa[lane + 64 * k]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    const float s2 = (m == 0.0f) ? 0.0f : m / 127.0f;
    if (threadIdx.x == 0) absmax_scale[group] = s2;
#pragma unroll
    for (int i = threadIdx.x; i < kGroupBlocks; i += NT) {
      const int64_t block = group * kGroupBlocks + i;
      if (block < args.nb) {
        const float a = sa[i];
        args.absmax[block] = a;
        absmax_q[block] = dq_code(a, s2);
      }
    }
  }
}

template <int BS, int QT, int W>
void launch_qdq_w(int64_t groups, QuantArgs args, int8_t *absmax_q, float *absmax_scale,
                  int64_t ngroups, hipStream_t stream) {
  hipLaunchKernelGGL((quantize_dq_kernel<BS, QT, W>), dim3((unsigned)groups), dim3(64 * W), 0,
                     stream, args, absmax_q, absmax_scale, ngroups);
}

template <int QT>
hipError_t launch_qdq(int blocksize, int64_t blocks, QuantArgs args, int8_t *absmax_q,
                      float *absmax_scale, int64_t ngroups, hipStream_t stream) {
  const bool wide = ngroups <= 256;
  switch (blocksize) {
    case 64:
      launch_qdq_w<64, QT, 4>(blocks, args, absmax_q, absmax_scale, ngroups, stream);
      break;
    case 128:
      if (wide) launch_qdq_w<128, QT, 8>(blocks, args, absmax_q, absmax_scale, ngroups, stream);
      else launch_qdq_w<128, QT, 4>(blocks, args, absmax_q, absmax_scale, ngroups, stream);
      break;
    case 256:
      if (wide) launch_qdq_w<256, QT, 8>(blocks, args, absmax_q, absmax_scale, ngroups, stream);
      else launch_qdq_w<256, QT, 4>(blocks, args, absmax_q, absmax_scale, ngroups, stream);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
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

QuantArgs make_args(const uint16_t *w, int64_t n, int blocksize, int quant_type, uint8_t *packed,
                    float *absmax) {
  const CodeTables &t = code_tables(quant_type);
  QuantArgs args;
  args.w = w;
  args.packed = packed;
  args.absmax = absmax;
  args.n = n;
  args.nb = (n + blocksize - 1) / blocksize;
  const int E = blocksize / 64 > 32 ? blocksize / 64 : 32;
  const int64_t tile_elems = 64LL * E;
  args.ntiles = (n + tile_elems - 1) / tile_elems;
  for (int i = 0; i < kCells; ++i) {
    args.cell_thr[i] = t.cell_thr[i];
    args.cell_codes[i] = t.cell_codes[i];
  }
  return args;
}

}  // namespace

bool quantize_dq_fused(int blocksize, int blocksize2) {
  return blocksize2 == 256 && (blocksize == 64 || blocksize == 128 || blocksize == 256);
}

hipError_t launch_quantize_dq(const uint16_t *w, int64_t n, int blocksize, int quant_type,
                              uint8_t *packed, float *absmax, int8_t *absmax_q,
                              float *absmax_scale, hipStream_t stream) {
  if (!quantize_dq_fused(blocksize, 256)) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  const QuantArgs args = make_args(w, n, blocksize, quant_type, packed, absmax);
  // a workgroup per group of 256 blocks, at most kMaxDqGroups of them; each
  // then loops over every kMaxDqGroups-th group
  const int64_t ngroups = (args.nb + 255) / 256;
  const int64_t blocks = ngroups < kMaxDqGroups ? ngroups : kMaxDqGroups;
  return quant_type == kQuantFP4
             ? launch_qdq<kQuantFP4>(blocksize, blocks, args, absmax_q, absmax_scale, ngroups, stream)
             : launch_qdq<kQuantNF4>(blocksize, blocks, args, absmax_q, absmax_scale, ngroups, stream);
}

hipError_t launch_quantize(const uint16_t *w, int64_t n, int blocksize, int quant_type,
                           uint8_t *packed, float *absmax, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const QuantArgs args = make_args(w, n, blocksize, quant_type, packed, absmax);
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
