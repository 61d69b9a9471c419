// quantize.hip -- blockwise NF4/FP4 quantization on gfx950.
//
// [NF4 page, CSDN "bitsandbytes 是一个用于高效量化和加载大型语言模型（LLM）的开源库",
//  table 数学原理对比, rows 缩放机制 (each block gets its own scale max|x|,
//  values normalised into [-1, 1]) and 量化目标 (nearest code value);
//  repo page ossradar.top bitsandbytes, release notes 0.49.2 (1-D blocksize 64
//  default, 32/128 also used; bs 64 on wave64 CDNA) and 0.50.2 (mask the absmax
//  store of the partial last block).]
//
// Layout of the work. Chunk c is elements [512 c, 512 c + 512); lane l owns
// 512 c + 8 l .. +7 (one 16-byte load, one 4-byte store of the packed
// codes). For bs <= 512 a block is bs / 8 neighbouring lanes of one chunk,
// and each wave walks its own sequence of chunks with kInFlight of them
// loaded ahead in a rotating register window (the load of a slot's next chunk
// is issued as soon as the slot has been encoded). Larger blocks take tiles of
// bs / 64 elements per lane, two tiles in flight per wave. With double
// quantization at bs 64/128/256 one launch also quantizes the scales: a
// workgroup owns each group of 256 blocks and meets its scales in LDS.
//
// Per element: s = x / a and the nearest code value. s is q0 = x * RN(1/a):
// that gives the same NF4 code as the correctly rounded RN(x/a) for every
// bf16 (x, a) pair (checked exhaustively over all significand/exponent
// classes); FP4 adds the residual correction q1 = q0 + (x - q0 a) RN(1/a)
// with two fmas, which equals RN(x/a) wherever the result is normal. Both
// hold while 1/a, the product and the residual stay normal, i.e. for a in
// [2^-100, 2^120). a is a bf16 value, so there RN(1/a) is the correctly
// rounded reciprocal of its significand (a 128-entry table, built on the host
// with IEEE division) times a power of two. Blocks outside that range (and
// all-zero blocks) first scale x and a by the power of two 2^sh that brings a
// into [1, 2): x / a is unchanged, the same arithmetic then holds, and RN(1/a)
// of the scaled a is an IEEE division. The choice is made per chunk for the
// whole wave (a ballot), so the common case runs without the scaling.
//
// The code of s is read from a 33-cell lookup in LDS (see cell_of), whose
// entry holds the one decision threshold that can fall inside the cell and
// the codes on either side of it; one compare and one byte-select move the
// code into place in the output word.
#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kThreads = 256;

// One tensor of a launch. group_begin: its first group of 256 blocks in the
// launch's group numbering (fused double quantization).
struct QTensor {
  const uint16_t *w;
  uint8_t *packed;
  float *absmax;
  int8_t *absmax_q;
  float *absmax_scale;
  int64_t n;
  int64_t nb;
  int64_t group_begin;
};

constexpr int kMaxQGroup = 16;

struct QuantArgs {
  QTensor t[kMaxQGroup];  // the single-tensor kernels use t[0]
  int32_t count;
  int64_t total_groups;
  int64_t ntiles;
  float cell_thr[kCells];
  uint32_t cell_codes[kCells];
  // bits of RN(1 / (1 + k/128)) plus 127 << 23, k = 0..127
  uint32_t recip[128];
};

template <int QT>
__device__ __forceinline__ float normalise(float x, float a, float r) {
  const float q0 = x * r;
  if (QT == kQuantNF4) return q0;
  const float e = __builtin_fmaf(-q0, a, x);
  return __builtin_fmaf(e, r, q0);
}

// Cell lookup: t = 2^23 + RN(128 s + 128) (one fma, the integer exact); its
// representation's low bits masked to a multiple of 8 are the byte offset of
// 8-byte entry floor(RN(128 s + 128) / 8). An entry holds a threshold and the
// codes below / above it, pre-placed as bytes: below, above in bytes 0, 1
// (low nibble) and below << 4, above << 4 in bytes 2, 3 (high nibble). Any bit
// pattern of t (a NaN from non-finite input included) stays inside the 64
// entries.
constexpr int kLutSize = 64;

__device__ __forceinline__ uint2 cell_of(float s, const uint2 *lut) {
  const float t = __builtin_fmaf(s, 128.0f, 8388736.0f);  // 2^23 + 128
  return *reinterpret_cast<const uint2 *>(reinterpret_cast<const char *>(lut) +
                                          (__float_as_uint(t) & 0x1f8u));
}

// Byte J of acc = (s > threshold) ? byte SRC + 1 : byte SRC of the entry's
// codes; J = 0 clears the other bytes, later J keep them. One compare and
// one byte-select (SDWA) per code.
template <int J, int SRC>
__device__ __forceinline__ void put_code(uint32_t &acc, float s, uint2 e) {
  const float thr = __uint_as_float(e.x);
  if constexpr (J == 0) {
    asm(
        "v_cmp_gt_f32 vcc, %1, %2\n\t"
        "s_nop 1\n\t"
        "v_cndmask_b32_sdwa %0, %3, %3, vcc dst_sel:BYTE_0 dst_unused:UNUSED_PAD "
        "src0_sel:BYTE_%4 src1_sel:BYTE_%5"
        : "=v"(acc)
        : "v"(s), "v"(thr), "v"(e.y), "n"(SRC), "n"(SRC + 1)
        : "vcc");
  } else {
    asm(
        "v_cmp_gt_f32 vcc, %1, %2\n\t"
        "s_nop 1\n\t"
        "v_cndmask_b32_sdwa %0, %3, %3, vcc dst_sel:BYTE_%6 dst_unused:UNUSED_PRESERVE "
        "src0_sel:BYTE_%4 src1_sel:BYTE_%5"
        : "+v"(acc)
        : "v"(s), "v"(thr), "v"(e.y), "n"(SRC), "n"(SRC + 1), "n"(J)
        : "vcc");
  }
}

// Codes of 8 elements. FAST: a in [2^-100, 2^120) and r = RN(1/a).
// Otherwise x and a are first scaled by 2^sh (exact) with a * 2^sh in [1, 2).
template <int QT, bool FAST>
__device__ __forceinline__ uint32_t encode8(const uint32_t d[4], float a, float r,
                                            const uint2 *lut) {
  int sh = 0;
  if (!FAST) {
    sh = 1 - __builtin_amdgcn_frexp_expf(a);
    a = __builtin_amdgcn_ldexpf(a, sh);
    r = (a == 0.0f) ? 0.0f : 1.0f / a;
  }
  uint32_t hi, lo;  // codes of the even / odd elements, as high / low nibbles
#define NF4_ENCODE_PAIR(J)                                     \
  {                                                            \
    float x0 = __uint_as_float(d[J] << 16);                    \
    float x1 = __uint_as_float(d[J] & 0xffff0000u);            \
    if (!FAST) {                                               \
      x0 = __builtin_amdgcn_ldexpf(x0, sh);                    \
      x1 = __builtin_amdgcn_ldexpf(x1, sh);                    \
    }                                                          \
    const float s0 = normalise<QT>(x0, a, r);                  \
    const float s1 = normalise<QT>(x1, a, r);                  \
    put_code<J, 2>(hi, s0, cell_of(s0, lut));                  \
    put_code<J, 0>(lo, s1, cell_of(s1, lut));                  \
  }
  // d[j] holds elements 2j (low half) and 2j+1 (high half): byte j of the
  // output is code(2j) << 4 | code(2j+1)
  NF4_ENCODE_PAIR(0)
  NF4_ENCODE_PAIR(1)
  NF4_ENCODE_PAIR(2)
  NF4_ENCODE_PAIR(3)
#undef NF4_ENCODE_PAIR
  return hi | lo;
}

// RN(1/a) for a block whose absmax has bf16 bits m, from the significand
// table; true when a lies in [2^-100, 2^120), where that value is exact.
__device__ __forceinline__ bool block_recip(uint32_t m, const uint32_t *recip, float &r) {
  r = __uint_as_float(recip[m & 0x7fu] - ((m << 16) & 0x7f800000u));
  return m - 0x0d80u < 0x6e00u;
}

__device__ __forceinline__ uint32_t absmax_bits16(const uint32_t d[4]) {
  u16x2 m = __builtin_bit_cast(u16x2, d[0] & 0x7fff7fffu);
#pragma unroll
  for (int j = 1; j < 4; ++j)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, d[j] & 0x7fff7fffu));
  return m.x > m.y ? m.x : m.y;
}

// Maximum over aligned groups of G lanes, every lane of a group gets it:
// DPP for partners within a 16-lane row, lane shuffles beyond.
template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t m) {
  uint32_t o;
  if (G >= 2) {
    o = __builtin_amdgcn_update_dpp(0u, m, 0xb1, 0xf, 0xf, false);  // quad_perm 1,0,3,2
    m = m > o ? m : o;
  }
  if (G >= 4) {
    o = __builtin_amdgcn_update_dpp(0u, m, 0x4e, 0xf, 0xf, false);  // quad_perm 2,3,0,1
    m = m > o ? m : o;
  }
  if (G >= 8) {
    o = __builtin_amdgcn_update_dpp(0u, m, 0x141, 0xf, 0xf, false);  // row_half_mirror
    m = m > o ? m : o;
  }
  if (G >= 16) {
    o = __builtin_amdgcn_update_dpp(0u, m, 0x140, 0xf, 0xf, false);  // row_mirror
    m = m > o ? m : o;
  }
#pragma unroll
  for (int off = 16; off < G; off <<= 1) {
    o = __shfl_xor(m, off, 64);
    m = m > o ? m : o;
  }
  return m;
}

// Codes of one lane's 8 elements given the block's absmax bits m.
template <int QT>
__device__ __forceinline__ uint32_t encode_lane(const uint32_t d[4], uint32_t m,
                                                const uint2 *lut, const uint32_t *recip) {
  float r;
  const bool fast = block_recip(m, recip, r);
  const float a = bf16_bits_to_f32(m);
  if (__builtin_amdgcn_ballot_w64(!fast) == 0) return encode8<QT, true>(d, a, r, lut);
  return encode8<QT, false>(d, a, 0.0f, lut);
}

// Packed codes of elements e0 .. e0 + 7; in a ragged tail the nibbles of
// missing elements are cleared and only the bytes that exist (ceil(n/2) in
// total) are written.
__device__ __forceinline__ void store_codes(const QTensor &T, int64_t e0, uint32_t word) {
  if (e0 + 8 <= T.n) {
    *reinterpret_cast<uint32_t *>(T.packed + e0 / 2) = word;
  } else if (e0 < T.n) {
    const int64_t valid = T.n - e0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (2 * b >= valid) break;
      uint32_t byte = (word >> (8 * b)) & 0xffu;
      if (2 * b + 1 >= valid) byte &= 0xf0u;
      T.packed[e0 / 2 + b] = (uint8_t)byte;
    }
  }
}

// The codes of one chunk: a whole chunk (the test is wave-uniform) stores
// through the chunk's base address plus a lane offset; the ragged last chunk
// goes element-wise.
__device__ __forceinline__ void store_chunk(const QTensor &T, int64_t chunk, int lane,
                                            uint32_t word) {
  if (chunk * 512 + 512 <= T.n) {
    uint32_t *base = reinterpret_cast<uint32_t *>(T.packed + chunk * 256);
    base[lane] = word;
  } else {
    store_codes(T, chunk * 512 + 8 * lane, word);
  }
}

// Zero the elements at or past n among a lane's 8 (d holds e0 .. e0 + 7).
__device__ __forceinline__ void clear_tail(uint32_t (&d)[4], int64_t e0, int64_t n) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (e0 + 2 * j >= n) d[j] = 0u;
    else if (e0 + 2 * j + 1 >= n) d[j] &= 0xffffu;
  }
}

__device__ __forceinline__ void load_tables(uint2 *lut, uint32_t *recip, const QuantArgs &args) {
  if (threadIdx.x < kLutSize) {
    const int c = threadIdx.x < kCells ? threadIdx.x : kCells - 1;
    lut[threadIdx.x] = make_uint2(__float_as_uint(args.cell_thr[c]), args.cell_codes[c]);
  }
  if (threadIdx.x < 128) recip[threadIdx.x] = args.recip[threadIdx.x];
  __syncthreads();
}

// ---- blocks of at most 512 elements: the chunk pipeline ------------------
constexpr int kInFlight = 4;

// Loads of chunk `chunk` through a buffer resource whose range is the chunk's
// bytes rounded up to whole 16-byte granules: granules past the end (and
// every granule of a chunk past the end) read as 0 without touching memory.
__device__ __forceinline__ void load_chunk(uint32_t (&d)[4], const QTensor &T, int64_t chunk,
                                           int lane) {
  const int64_t c0 = chunk * 512;
  const int64_t rem = T.n - c0;
  const int64_t valid = rem < 512 ? (rem > 0 ? rem : 0) : 512;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(T.w + (c0 < T.n ? c0 : 0)), (short)0,
      (int)((2 * valid + 15) & ~(int64_t)15), 0x00020000);
  const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane, 0, 0));
  d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
}

// Absmax bits (returned) and packed codes of one chunk.
template <int BS, int QT>
__device__ __forceinline__ uint32_t encode_chunk(uint32_t (&d)[4], const QTensor &T,
                                                 int64_t chunk, int lane, const uint2 *lut,
                                                 const uint32_t *recip, uint32_t &word) {
  if (chunk * 512 + 512 > T.n) clear_tail(d, chunk * 512 + 8 * lane, T.n);
  const uint32_t m = group_max<BS / 8>(absmax_bits16(d));
  word = encode_lane<QT>(d, m, lut, recip);
  return m;
}

// bs <= 512: wave w of the grid takes chunks w, w + nwaves, w + 2 nwaves, ...
template <int BS, int QT>
__global__ __launch_bounds__(kThreads) void quantize_chunks_kernel(QuantArgs args) {
  constexpr int G = BS / 8;
  __shared__ uint2 lut[kLutSize];
  __shared__ uint32_t recip[128];
  load_tables(lut, recip, args);
  const int lane = threadIdx.x & 63;
  // wave-uniform (readfirstlane), so chunk addresses and buffer resources
  // live in scalar registers
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  const QTensor &T = args.t[0];
  const int64_t nchunks = (T.n + 511) / 512;
  const int64_t nseq = wave < nchunks ? (nchunks - 1 - wave) / nwaves + 1 : 0;

  // Loads are issued unconditionally (a chunk past the end has an empty
  // range), so the number of loads in flight is the same on every path and
  // each encode waits for its own chunk only.
  uint32_t d[kInFlight][4];
#pragma unroll
  for (int u = 0; u < kInFlight; ++u) load_chunk(d[u], T, wave + u * nwaves, lane);
  for (int64_t i0 = 0; i0 < nseq; i0 += kInFlight) {
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int64_t i = i0 + u;
      if (i >= nseq) break;
      const int64_t chunk = wave + i * nwaves;
      uint32_t word;
      const uint32_t m = encode_chunk<BS, QT>(d[u], T, chunk, lane, lut, recip, word);
      load_chunk(d[u], T, chunk + kInFlight * nwaves, lane);
      store_chunk(T, chunk, lane, word);
      const int64_t block = (chunk * 512 + 8 * lane) / BS;
      if (lane % G == 0 && block < T.nb) T.absmax[block] = bf16_bits_to_f32(m);
    }
  }
}

// ---- blocks of more than 512 elements: whole tiles -----------------------
// A tile is 64 * E elements, E = bs / 64 per lane in E / 8 chunks (chunk c of
// the tile is its elements [512 c, 512 c + 512)); a block is bs / 512 chunks.
template <int BS>
struct TileShape {
  static constexpr int E = BS / 64;
  static constexpr int CH = E / 8;      // chunks per lane (per tile)
  static constexpr int kTile = 64 * E;  // elements per tile
};

// Loads of one tile, with the same range rule as load_chunk.
template <int BS>
__device__ __forceinline__ void load_tile(uint32_t (&d)[TileShape<BS>::CH][4],
                                          const QTensor &T, int64_t tile, int lane) {
  constexpr int CH = TileShape<BS>::CH, kTile = TileShape<BS>::kTile;
  const int64_t t0 = tile * kTile;
  const int64_t rem = T.n - t0;
  const int64_t valid = rem < kTile ? (rem > 0 ? rem : 0) : kTile;
  const uint32_t bytes = (uint32_t)((2 * valid + 15) & ~(int64_t)15);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(T.w + (t0 < T.n ? t0 : 0)), (short)0, (int)bytes, 0x00020000);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const uint4 v = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(1024 * c + 16 * lane), 0, 0));
    d[c][0] = v.x; d[c][1] = v.y; d[c][2] = v.z; d[c][3] = v.w;
  }
}

template <int BS, int QT>
__device__ __forceinline__ void encode_tile(uint32_t (&d)[TileShape<BS>::CH][4],
                                            const QTensor &T, int64_t tile, int lane,
                                            const uint2 *lut, const uint32_t *recip) {
  constexpr int CH = TileShape<BS>::CH, kTile = TileShape<BS>::kTile;
  constexpr int CPB = BS / 512;  // chunks per block
  const int64_t t0 = tile * kTile;
  if (t0 + kTile > T.n) {
#pragma unroll
    for (int c = 0; c < CH; ++c) clear_tail(d[c], t0 + 512 * c + 8 * lane, T.n);
  }
#pragma unroll
  for (int j = 0; j < CH / CPB; ++j) {
    uint32_t m = 0;
#pragma unroll
    for (int c = j * CPB; c < (j + 1) * CPB; ++c) {
      const uint32_t mc = absmax_bits16(d[c]);
      m = m > mc ? m : mc;
    }
    m = group_max<64>(m);
    const int64_t block = t0 / BS + j;
    if (lane == 0 && block < T.nb) T.absmax[block] = bf16_bits_to_f32(m);
#pragma unroll
    for (int c = j * CPB; c < (j + 1) * CPB; ++c)
      store_codes(T, t0 + 512 * c + 8 * lane, encode_lane<QT>(d[c], m, lut, recip));
  }
}

template <int BS, int QT>
__global__ __launch_bounds__(kThreads) void quantize_tiles_kernel(QuantArgs args) {
  constexpr int CH = TileShape<BS>::CH;
  __shared__ uint2 lut[kLutSize];
  __shared__ uint32_t recip[128];
  load_tables(lut, recip, args);

  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  const QTensor &T = args.t[0];

  uint32_t da[CH][4], db[CH][4];
  int64_t tile = wave;
  if (tile < args.ntiles) load_tile<BS>(da, T, tile, lane);
  for (; tile < args.ntiles; tile += 2 * nwaves) {
    const int64_t t1 = tile + nwaves;
    load_tile<BS>(db, T, t1 < args.ntiles ? t1 : tile, lane);
    encode_tile<BS, QT>(da, T, tile, lane, lut, recip);
    if (t1 >= args.ntiles) break;
    const int64_t t2 = t1 + nwaves;
    load_tile<BS>(da, T, t2 < args.ntiles ? t2 : t1, lane);
    encode_tile<BS, QT>(db, T, t1, lane, lut, recip);
  }
}

// ---- quantization with double quantization in one pass -------------------
// [NF4 page, CSDN "bitsandbytes 是一个用于高效量化和加载大型语言模型（LLM）的开源库",
// table 实际性能差异, row 训练稳定性（QLoRA）: the block scales are quantized
// again with INT8]. A workgroup owns one group of 256 blocks at a time and
// each of its W waves a contiguous run of CPW chunks of it, walked with the
// chunk pipeline (the window runs on into the workgroup's next group). The
// scales of the group meet in LDS, where every wave takes their maximum, and
// the threads then store the fp32 absmax and the int8 code of one block each,
// so both stores are coalesced. The arithmetic is that of the separate
// double-quant kernel: m = fmaxf over the group, s2 = RN(m / 127) (0 for
// m = 0), q = clamp(rint(RN(a / s2)), -127, 127), ties to even.
__device__ __forceinline__ int8_t dq_code(float a, float s2) {
  if (s2 == 0.0f) return 0;
  float r = __builtin_rintf(a / s2);
  r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
  return (int8_t)(int)r;
}

constexpr int kGroupBlocks = 256;
constexpr int64_t kMaxDqGroups = 256 * 64;  // workgroups of one fused launch

template <int BS, int W>
struct DqShape {
  static constexpr int CPG = kGroupBlocks * BS / 512;  // chunks per group
  static constexpr int CPW = CPG / W;                  // chunks per wave
};

// The launch may hold several tensors (one group numbering over all of
// them); a group never spans two tensors.
template <int BS, int QT, int W, bool MULTI>
__global__ __launch_bounds__(64 * W) void quantize_dq_kernel(QuantArgs args) {
  constexpr int CPG = DqShape<BS, W>::CPG, CPW = DqShape<BS, W>::CPW;
  static_assert(BS <= 512 && CPW % kInFlight == 0, "whole windows per wave and group");
  constexpr int G = BS / 8;  // lanes per block

  __shared__ uint2 lut[kLutSize];
  __shared__ uint32_t recip[128];
  __shared__ float sabs[2][kGroupBlocks];
  load_tables(lut, recip, args);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
  const int64_t ngroups = args.total_groups;
  // i-th chunk of this wave: group blockIdx.x + (i / CPW) * gridDim.x of the
  // launch, chunk wave * CPW + i % CPW of that group
  const int64_t my_groups =
      blockIdx.x < ngroups ? (ngroups - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  const int64_t nseq = my_groups * CPW;
  // tensor of launch group lg and the group's index within it (a group past
  // the last one maps past the last tensor's end: its loads read nothing).
  // The tensors' first groups are read once into scalar registers (unused
  // entries hold INT64_MAX), so a lookup is a short compare chain.
  // (a launch of one tensor skips all of this: its tensor is fixed, so its
  // fields load once)
  constexpr int kT = MULTI ? kMaxQGroup : 1;
  int64_t gb[kT];
#pragma unroll
  for (int k = 0; k < kT; ++k) gb[k] = MULTI ? args.t[k].group_begin : 0;
  auto locate = [&](int64_t lg, int &ti, int64_t &g) {
    int t = 0;
#pragma unroll
    for (int k = 1; k < kT; ++k) t = gb[k] <= lg ? k : t;
    ti = t;
    g = lg - gb[t];
  };
  // window i0 (kInFlight chunks, never across two groups): its tensor and the
  // group's first chunk of this wave
  auto window = [&](int64_t i0, int &ti) -> int64_t {
    int64_t g;
    locate((int64_t)blockIdx.x + (i0 / CPW) * gridDim.x, ti, g);
    return g * CPG + wave * CPW + i0 % CPW;
  };

  // loads are unconditional: past the last group a chunk has an empty range
  uint32_t d[kInFlight][4];
  int tc;
  int64_t cc = window(0, tc);
#pragma unroll
  for (int u = 0; u < kInFlight; ++u) load_chunk(d[u], args.t[tc], cc + u, lane);
  for (int64_t i0 = 0; i0 < nseq; i0 += kInFlight) {
    const int64_t it = i0 / CPW;
    float *sa = sabs[it & 1];
    int tn;
    const int64_t cn = window(i0 + kInFlight, tn);
    const QTensor &T = args.t[tc];
    const QTensor &Tn = args.t[tn];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int64_t chunk = cc + u;
      uint32_t word;
      const uint32_t m = encode_chunk<BS, QT>(d[u], T, chunk, lane, lut, recip, word);
      load_chunk(d[u], Tn, cn + u, lane);
      store_chunk(T, chunk, lane, word);
      if (lane % G == 0)
        sa[((wave * CPW + (i0 + u) % CPW) * 512 + 8 * lane) / BS] = bf16_bits_to_f32(m);
    }
    const int t_done = tc;
    tc = tn;
    cc = cn;
    if ((i0 + kInFlight) % CPW != 0) continue;
    // the group is complete: its scale maximum (blocks past n hold 0), taken by every wave
    const QTensor &Td = args.t[t_done];
    const int64_t group = (int64_t)blockIdx.x + it * gridDim.x - gb[t_done];
    __syncthreads();
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < kGroupBlocks / 64; ++k) mx = fmaxf(mx, sa[lane + 64 * k]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    const float s2 = (mx == 0.0f) ? 0.0f : mx / 127.0f;
    if (threadIdx.x == 0) Td.absmax_scale[group] = s2;
#pragma unroll
    for (int i = threadIdx.x; i < kGroupBlocks; i += 64 * W) {
      const int64_t block = group * kGroupBlocks + i;
      if (block < Td.nb) {
        const float a = sa[i];
        Td.absmax[block] = a;
        Td.absmax_q[block] = dq_code(a, s2);
      }
    }
  }
}

template <int BS, int QT, int W>
void launch_qdq_w(int64_t groups, const QuantArgs &args, hipStream_t stream) {
  if (args.count > 1)
    hipLaunchKernelGGL((quantize_dq_kernel<BS, QT, W, true>), dim3((unsigned)groups), dim3(64 * W),
                       0, stream, args);
  else
    hipLaunchKernelGGL((quantize_dq_kernel<BS, QT, W, false>), dim3((unsigned)groups),
                       dim3(64 * W), 0, stream, args);
}

// Waves per group: the fewest of 4, 8, 16 that give the launch at least
// kWantWaves waves (8 per SIMD), while every wave keeps at least one whole
// window of chunks.
constexpr int64_t kWantWaves = 256 * 4 * 8;

template <int BS, int QT>
void launch_qdq_bs(int64_t blocks, const QuantArgs &args, hipStream_t stream) {
  constexpr int kMaxW = DqShape<BS, 1>::CPG / kInFlight >= 16 ? 16 : DqShape<BS, 1>::CPG / kInFlight;
  const int64_t ngroups = args.total_groups;
  if (ngroups * 4 >= kWantWaves || kMaxW < 8)
    launch_qdq_w<BS, QT, 4>(blocks, args, stream);
  else if (ngroups * 8 >= kWantWaves || kMaxW < 16)
    launch_qdq_w<BS, QT, (kMaxW < 8 ? 4 : 8)>(blocks, args, stream);
  else
    launch_qdq_w<BS, QT, (kMaxW < 8 ? 4 : (kMaxW < 16 ? 8 : 16))>(blocks, args, stream);
}

template <int QT>
hipError_t launch_qdq(int blocksize, int64_t blocks, const QuantArgs &args, hipStream_t stream) {
  switch (blocksize) {
    case 64: launch_qdq_bs<64, QT>(blocks, args, stream); break;
    case 128: launch_qdq_bs<128, QT>(blocks, args, stream); break;
    case 256: launch_qdq_bs<256, QT>(blocks, args, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int QT>
hipError_t launch_qt(int blocksize, dim3 grid, QuantArgs args, hipStream_t stream) {
  switch (blocksize) {
#define NF4_QCCASE(BSV)                                                                         \
  case BSV:                                                                                     \
    hipLaunchKernelGGL((quantize_chunks_kernel<BSV, QT>), grid, dim3(kThreads), 0, stream, args); \
    break;
#define NF4_QTCASE(BSV)                                                                        \
  case BSV:                                                                                    \
    hipLaunchKernelGGL((quantize_tiles_kernel<BSV, QT>), grid, dim3(kThreads), 0, stream, args); \
    break;
    NF4_QCCASE(32)
    NF4_QCCASE(64)
    NF4_QCCASE(128)
    NF4_QCCASE(256)
    NF4_QCCASE(512)
    NF4_QTCASE(1024)
    NF4_QTCASE(2048)
    NF4_QTCASE(4096)
#undef NF4_QCCASE
#undef NF4_QTCASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Arguments of a launch over `count` tensors that share blocksize and quant type.
QuantArgs make_args(int count, const QuantTensorDesc *ts, int blocksize, int quant_type) {
  const CodeTables &t = code_tables(quant_type);
  QuantArgs args;
  args.count = count;
  int64_t groups = 0;
  for (int i = 0; i < count; ++i) {
    QTensor &T = args.t[i];
    T.w = ts[i].w;
    T.packed = ts[i].packed;
    T.absmax = ts[i].absmax;
    T.absmax_q = ts[i].absmax_q;
    T.absmax_scale = ts[i].absmax_scale;
    T.n = ts[i].n;
    T.nb = (T.n + blocksize - 1) / blocksize;
    T.group_begin = groups;
    groups += (T.nb + kGroupBlocks - 1) / kGroupBlocks;
  }
  args.total_groups = groups;
  for (int i = count; i < kMaxQGroup; ++i) {
    args.t[i] = args.t[0];
    args.t[i].group_begin = INT64_MAX;  // never found by a group lookup
  }
  const int64_t tile_elems = blocksize > 512 ? blocksize : 512;
  args.ntiles = count > 0 ? (args.t[0].n + tile_elems - 1) / tile_elems : 0;
  for (int i = 0; i < kCells; ++i) {
    args.cell_thr[i] = t.cell_thr[i];
    args.cell_codes[i] = t.cell_codes[i];
  }
  for (int k = 0; k < 128; ++k) {
    // 1 + k/128 is exact in fp32 and the host division is IEEE (correctly rounded)
    volatile float den = 1.0f + (float)k / 128.0f;
    const float rk = 1.0f / den;
    uint32_t bits;
    __builtin_memcpy(&bits, &rk, 4);
    args.recip[k] = bits + (127u << 23);
  }
  return args;
}

// ---- general inputs: bf16 / fp16 / fp32 elements, row-strided matrices ---
// [repo page, release notes 0.49.2: quantize accepts non-contiguous tensors;
//  usage page, Core Usage 3: Linear4bit quantizes fp16 or bf16 weights.]
// The flattened row-major element e of a [rows, cols] matrix with row stride
// ld lives at e + (e / cols) (ld - cols); with a stride, cols % 8 == 0, so the
// 8 elements a lane takes lie in one row. Each element is widened exactly to
// fp32, s = x / a is the correctly rounded IEEE quotient (no reciprocal
// shortcut: that equality is shown for bf16 pairs only), and its code comes
// from the same cell lookup, which is exact for every fp32 s in [-1, 1].
// A wave owns tiles of max(bs, 512) elements; lane l takes elements 512 j +
// 8 l .. + 7 of its tile.
template <int DT>
__device__ __forceinline__ void load8_elems(float (&x)[8], const void *w, int64_t off, int valid) {
  if (DT == kFP32) {
    const float *p = static_cast<const float *>(w) + off;
    if (valid == 8) {
      const float4 a = *reinterpret_cast<const float4 *>(p);
      const float4 b = *reinterpret_cast<const float4 *>(p + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = j < valid ? p[j] : 0.0f;
    }
  } else {
    const uint16_t *p = static_cast<const uint16_t *>(w) + off;
    uint16_t h[8];
    if (valid == 8) {
      const uint4 v = *reinterpret_cast<const uint4 *>(p);
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[2 * j] = (uint16_t)(d[j] & 0xffffu);
        h[2 * j + 1] = (uint16_t)(d[j] >> 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = j < valid ? p[j] : (uint16_t)0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = DT == kFP16 ? widen16<kFP16>(h[j]) : widen16<kBF16>(h[j]);
  }
}

// code of s through the cell lookup: the one threshold inside s's cell
// decides between the codes below and above it
__device__ __forceinline__ uint32_t code_of(float s, const uint2 *lut) {
  const uint2 e = cell_of(s, lut);
  return s > __uint_as_float(e.x) ? (e.y >> 8) & 0xfu : e.y & 0xfu;
}

template <int DT, int BS>
__global__ __launch_bounds__(kThreads) void quantize_generic_kernel(
    const void *w, int64_t n, int64_t cols, int64_t ld, uint8_t *packed, float *absmax,
    int64_t ntiles, QuantArgs args) {
  constexpr int kTile = BS > 512 ? BS : 512;
  constexpr int P = kTile / 512;   // 8-element pieces per lane
  constexpr int G = BS >= 512 ? 64 : BS / 8;  // lanes per block within a piece
  __shared__ uint2 lut[kLutSize];
  __shared__ uint32_t recip[128];
  load_tables(lut, recip, args);
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t nb = (n + BS - 1) / BS;
  const bool strided = ld != cols;
  for (int64_t tile = wave; tile < ntiles; tile += nwaves) {
    float x[P][8];
    int64_t e0[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
      e0[j] = tile * kTile + 512 * j + 8 * lane;
      const int64_t rem = n - e0[j];
      const int valid = rem >= 8 ? 8 : (rem > 0 ? (int)rem : 0);
      int64_t off = e0[j];
      if (strided && valid > 0) {
        const int64_t row = e0[j] / cols;
        off = row * ld + (e0[j] - row * cols);
      }
      if (valid > 0) load8_elems<DT>(x[j], w, off, valid);
      else {
#pragma unroll
        for (int k = 0; k < 8; ++k) x[j][k] = 0.0f;
      }
    }
    // block maxima: within a piece for bs <= 512, over the whole tile beyond
    float m[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
      float v = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) v = fmaxf(v, fabsf(x[j][k]));
      m[j] = v;
    }
    if (BS > 512) {
      float v = m[0];
#pragma unroll
      for (int j = 1; j < P; ++j) v = fmaxf(v, m[j]);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
#pragma unroll
      for (int j = 0; j < P; ++j) m[j] = v;
      if (lane == 0 && tile < nb) absmax[tile] = v;
    } else {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        // |x| >= 0, so the fp32 bit patterns order like the values
        m[j] = __uint_as_float(group_max<G>(__float_as_uint(m[j])));
        const int64_t b = e0[j] / BS;
        if (lane % G == 0 && b < nb) absmax[b] = m[j];
      }
    }
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const float a = m[j];
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float sv = a == 0.0f ? 0.0f : x[j][k] / a;
        const uint32_t c = code_of(sv, lut);
        // byte k / 2: element 2i in the high nibble, 2i + 1 in the low one
        word |= c << (8 * (k >> 1) + ((k & 1) ? 0 : 4));
      }
      QTensor T;
      T.packed = packed;
      T.n = n;
      store_codes(T, e0[j], word);
    }
  }
}

template <int DT>
hipError_t launch_generic_dt(const void *w, int64_t n, int64_t cols, int64_t ld, int blocksize,
                             uint8_t *packed, float *absmax, int64_t ntiles, dim3 grid,
                             const QuantArgs &args, hipStream_t stream) {
  switch (blocksize) {
#define NF4_QGCASE(BSV)                                                                          \
  case BSV:                                                                                      \
    hipLaunchKernelGGL((quantize_generic_kernel<DT, BSV>), grid, dim3(kThreads), 0, stream, w, n, \
                       cols, ld, packed, absmax, ntiles, args);                                  \
    break;
    NF4_QGCASE(32)
    NF4_QGCASE(64)
    NF4_QGCASE(128)
    NF4_QGCASE(256)
    NF4_QGCASE(512)
    NF4_QGCASE(1024)
    NF4_QGCASE(2048)
    NF4_QGCASE(4096)
#undef NF4_QGCASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool quantize_dq_fused(int blocksize, int blocksize2) {
  return blocksize2 == 256 && (blocksize == 64 || blocksize == 128 || blocksize == 256);
}

int quantize_max_group() { return kMaxQGroup; }

hipError_t launch_quantize_dq(int count, const QuantTensorDesc *ts, int blocksize,
                              int quant_type, hipStream_t stream) {
  if (!quantize_dq_fused(blocksize, 256) || count > kMaxQGroup) return hipErrorInvalidValue;
  QuantTensorDesc live[kMaxQGroup];
  int nl = 0;
  for (int i = 0; i < count; ++i)
    if (ts[i].n > 0) live[nl++] = ts[i];
  if (nl == 0) return hipSuccess;
  const QuantArgs args = make_args(nl, live, blocksize, quant_type);
  // a workgroup per group of 256 blocks, at most kMaxDqGroups of them; each
  // then loops over every kMaxDqGroups-th group
  const int64_t ngroups = args.total_groups;
  const int64_t blocks = ngroups < kMaxDqGroups ? ngroups : kMaxDqGroups;
  return quant_type == kQuantFP4 ? launch_qdq<kQuantFP4>(blocksize, blocks, args, stream)
                                 : launch_qdq<kQuantNF4>(blocksize, blocks, args, stream);
}

hipError_t launch_quantize(const uint16_t *w, int64_t n, int blocksize, int quant_type,
                           uint8_t *packed, float *absmax, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const QuantTensorDesc one{w, n, packed, absmax, nullptr, nullptr};
  const QuantArgs args = make_args(1, &one, blocksize, quant_type);
  // Enough waves to keep every CU's memory pipeline busy (about four chunks
  // or one tile per wave); each wave then strides over the rest.
  const int64_t waves_wanted = blocksize <= 512 ? (args.ntiles + 3) / 4 : args.ntiles;
  int64_t blocks = (waves_wanted + (kThreads / 64) - 1) / (kThreads / 64);
  const int64_t max_blocks = 256 * 16;
  if (blocks > max_blocks) blocks = max_blocks;
  dim3 grid((unsigned)blocks);
  return quant_type == kQuantFP4 ? launch_qt<kQuantFP4>(blocksize, grid, args, stream)
                                 : launch_qt<kQuantNF4>(blocksize, grid, args, stream);
}

}  // namespace nf4

namespace nf4 {

hipError_t launch_quantize_generic(const void *w, int w_dtype, int64_t rows, int64_t cols,
                                   int64_t ld, int blocksize, int quant_type, uint8_t *packed,
                                   float *absmax, hipStream_t stream) {
  const int64_t n = rows * cols;
  if (n == 0) return hipSuccess;
  const QuantTensorDesc one{nullptr, n, packed, absmax, nullptr, nullptr};
  const QuantArgs args = make_args(1, &one, blocksize, quant_type);
  const int64_t tile = blocksize > 512 ? blocksize : 512;
  const int64_t ntiles = (n + tile - 1) / tile;
  int64_t blocks = (ntiles + (kThreads / 64) - 1) / (kThreads / 64);
  if (blocks > 256 * 16) blocks = 256 * 16;
  const dim3 grid((unsigned)blocks);
  // one row (or a contiguous matrix) is its flattened self
  const int64_t c = rows > 1 ? cols : n, l = rows > 1 ? ld : n;
  if (w_dtype == kFP32)
    return launch_generic_dt<kFP32>(w, n, c, l, blocksize, packed, absmax, ntiles, grid, args,
                                    stream);
  if (w_dtype == kFP16)
    return launch_generic_dt<kFP16>(w, n, c, l, blocksize, packed, absmax, ntiles, grid, args,
                                    stream);
  return launch_generic_dt<kBF16>(w, n, c, l, blocksize, packed, absmax, ntiles, grid, args,
                                  stream);
}

}  // namespace nf4
