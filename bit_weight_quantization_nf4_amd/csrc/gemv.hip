// gemv.hip -- decode products y_i[M, N_i] = x_i[M, K_i] . bf16(dequant(W_i))^T
// for 1 <= M <= 16, one or several independent problems per launch, on gfx950
// matrix cores.
//
// [repo page ossradar.top bitsandbytes, release notes 0.50.0: 4-bit inference
//  at batch 1 uses a 4-bit GEMV, batches 2..64 a fused 4-bit dequantize + GEMM
//  in place of dequantize + F.linear; usage page icman.com.cn/news/48546,
//  "Configuration": weights are dequantized to the bf16 compute dtype before
//  the product.]
//
// Design (HBM-bound: every 4-bit weight is read once; x is tiny). Two
// kernels; a product takes the one its K decides, whatever it is grouped
// with, so its result does not depend on the grouping:
//  - K <= 6144 (gemv_xreg_kernel): a 16-wave workgroup per CU; wave w owns a
//    fixed slice of the 128-code chunks of K and holds x of that slice in
//    registers, loaded once per problem. Persistent workgroups walk work
//    items of 16 weight rows (32, with two accumulators per wave, in big
//    launches of short rows) with two register sets of item loads in turn,
//    so the codes and scales of the next item are in flight while the
//    current one is computed; the 16 partial tiles of an item are added in
//    wave order through LDS;
//  - longer K (gemv_kernel): work items of 16 (32 when there are enough) rows,
//    persistent workgroups of 8 waves that split K, x streamed with each
//    chunk, partial sums added in a fixed order through LDS;
//  - both run on v_mfma_f32_16x16x32_bf16 with x as the A operand (rows
//    m >= M only feed outputs that are never stored) and dequantized weights
//    as the B operand. Lane (n, kg) of the B operand needs 8 consecutive k
//    of weight row n, i.e. one 32-bit word of packed codes; a lane loads 16
//    bytes = 32 codes and feeds four MFMAs. The A operand is permuted the same
//    way, so the k order inside a chunk does not matter;
//  - dequantization goes through an LDS table indexed by a whole code BYTE:
//    entry e holds the fp32 code values of its two nibbles, so one 8-byte LDS
//    read serves two weights. The table is stored 32 times, interleaved so
//    that copy (lane % 32) sits in its own bank pair (entry e of copy c at
//    byte 256*e + 8*c): lookups never conflict, and the address is the code
//    byte moved into bits 15..8 of the lane's base by one v_perm_b32. Per two
//    weights: 1 perm, 1 LDS read, 2 multiplies by the block scale, 1
//    v_cvt_pk_bf16_f32 -- the same bf16 weights the dequantize kernel writes;
//  - an optional bf16 bias per output row (nf4_linear) is loaded at the start
//    of an item by the thread that stores that output, and added to its sum.
#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 128;                 // codes of one row per wave step
constexpr int kCopies = 32;                 // interleaved copies of the pair table
constexpr int kTableBytes = 256 * 256;      // 256 entries x 256-byte rows
constexpr int kMaxGroup = 16;
// Word 3 of a raw (untyped, unswizzled) buffer resource on gfx9, and an offset
// past every buffer's end.
constexpr int kBufferFlags = 0x00020000;
constexpr int kOutOfRange = 0x7fffffff;

struct GemvProblem {
  const uint16_t *x;
  const uint8_t *packed;
  void *y;
  const uint16_t *bias;  // [N] bf16 or null
  const float *absmax;
  const int8_t *absmax_q;
  const float *absmax_scale;
  int32_t N, K;
  int32_t log2_bs, log2_bs2;
  int32_t item_begin;  // first work item of this problem
};

struct GemvArgs {
  GemvProblem p[kMaxGroup];
  int32_t count;
  int32_t M;
  int32_t total_items;
  float value[16];
};

// 8 codes of one packed word -> 4 registers of bf16 pairs in k order (byte j
// holds element 2j in its high nibble and 2j+1 in its low nibble).
__device__ __forceinline__ bf16x8 dequant8(uint32_t word, float ap, const char *tbl,
                                           uint32_t lane_base) {
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // bytes of the address: [0] lane_base[0] (= 8 * copy), [1] code byte j, [2..3] zero
    const uint32_t addr = __builtin_amdgcn_perm(word, lane_base, 0x0c0c0000u | ((4u + j) << 8));
    const f32x2 c = *reinterpret_cast<const f32x2 *>(tbl + addr);
    out[j] = pack_bf16x2(c.x * ap, c.y * ap);
  }
  uint4 v = make_uint4(out[0], out[1], out[2], out[3]);
  return __builtin_bit_cast(bf16x8, v);
}

template <int NG, int CPW, bool DQ, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs args) {
  __shared__ __attribute__((aligned(16))) char lds[kTableBytes + kWaves * NG * 4 * 64 * 4];
  const char *tbl = lds;
  float *red = reinterpret_cast<float *>(lds + kTableBytes);  // [kWaves][NG][4][64]

  // Pair table, entry e = (value[e >> 4], value[e & 15]) at 256 e + 8 copy.
  // Consecutive lanes write consecutive copies (no bank conflicts); in pass i
  // every entry has e >> 4 == i.
  {
    const float lo = args.value[(threadIdx.x >> 5) & 15];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int idx = threadIdx.x + kThreads * i;  // e = idx / 32, copy = idx % 32
      const f32x2 v = {args.value[i], lo};
      *reinterpret_cast<f32x2 *>(lds + 256 * (idx >> 5) + 8 * (idx & 31)) = v;
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;  // B column (weight row in the group) / A row (m)
  const int kg = lane >> 4;  // which 32-code piece of the chunk
  const uint32_t lane_base = 8u * (uint32_t)(lane & (kCopies - 1));
  const int M = args.M;

  for (int item = blockIdx.x; item < args.total_items; item += gridDim.x) {
    int pi = 0;
    while (pi + 1 < args.count && args.p[pi + 1].item_begin <= item) ++pi;
    const GemvProblem &P = args.p[pi];
    const int N = P.N, K = P.K;
    const int row0 = (item - P.item_begin) * 16 * NG;
    const int nch = (K + kChunk - 1) / kChunk;
    const int c_begin = (wave * nch) / kWaves;
    const int c_end = ((wave + 1) * nch) / kWaves;
    const int kg_last = (K - (nch - 1) * kChunk) >> 5;  // valid pieces in the last chunk

    f32x4 acc[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the bias of the one output this thread writes at the end of the item
    // (NG * 256 <= kThreads), fetched now so its latency is hidden
    const bool has_bias = P.bias != nullptr;
    uint32_t bias_bits;
    {
      static_assert(NG * 4 * 64 <= kThreads, "one output per thread");
      const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
          (void *)P.bias, (short)0, has_bias ? 2 * N : 0, kBufferFlags);
      const int n = row0 + 16 * ((int)threadIdx.x / 256) + ((int)threadIdx.x & 15);
      bias_bits = __builtin_amdgcn_raw_buffer_load_b16(brs, 2 * n, 0, 0);
    }

    // Activations through a buffer resource: lanes whose row m >= M get an
    // out-of-range offset, which returns zeros without a memory access, so
    // only the M live rows of the A operand are fetched.
    const __amdgpu_buffer_rsrc_t xres =
        __builtin_amdgcn_make_buffer_rsrc((void *)P.x, (short)0, M * K * 2, kBufferFlags);
    const int xoff0 = nl < M ? (nl * K + 32 * kg) * 2 : kOutOfRange;
    bool row_ok[NG];
    const uint8_t *prow[NG];
    int64_t brow[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int row = row0 + 16 * g + nl;
      row_ok[g] = row < N;
      const int64_t e = (int64_t)(row_ok[g] ? row : N - 1) * K + 32 * kg;
      prow[g] = P.packed + e / 2;
      brow[g] = e;
    }

    for (int cb = c_begin; cb < c_end; cb += CPW) {
      // every load of the batch first (clamped, unconditional) ...
      uint4 xa[CPW][4];
      uint4 pw[CPW][NG];
      float sf[CPW][NG];
      int32_t sq[CPW][NG];
      bool ok[CPW];
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        int c = cb + i;
        ok[i] = c < c_end && (c < nch - 1 || kg < kg_last);
        if (c >= c_end) c = c_end - 1;
        // a piece past K (last chunk only) reads the chunk start instead
        const int kc = c * kChunk - ((c == nch - 1 && kg >= kg_last) ? 32 * kg : 0);
        const int xoff = xoff0 == kOutOfRange ? kOutOfRange : xoff0 + 2 * kc;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          xa[i][s] = __builtin_bit_cast(
              uint4, __builtin_amdgcn_raw_buffer_load_b128(
                         xres, (int)((uint32_t)xoff + 16u * s), 0, 0));
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          pw[i][g] = *reinterpret_cast<const uint4 *>(prow[g] + kc / 2);
          const int64_t b = (brow[g] + kc) >> P.log2_bs;
          if (DQ) {
            sq[i][g] = P.absmax_q[b];
            sf[i][g] = P.absmax_scale[b >> P.log2_bs2];
          } else {
            sq[i][g] = 1;
            sf[i][g] = P.absmax[b];
          }
        }
      }
      // ... then the arithmetic
#pragma unroll
      for (int i = 0; i < CPW; ++i)
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          float ap = DQ ? (float)sq[i][g] * sf[i][g] : sf[i][g];
          ap = (ok[i] && row_ok[g]) ? ap : 0.0f;
          const uint32_t words[4] = {pw[i][g].x, pw[i][g].y, pw[i][g].z, pw[i][g].w};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            bf16x8 b = dequant8(words[s], ap, tbl, lane_base);
            bf16x8 a = __builtin_bit_cast(bf16x8, xa[i][s]);
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[g], 0, 0, 0);
          }
        }
    }

    // Cross-wave reduction in a fixed order (the first barrier also fences
    // the previous item's reads of the buffer).
    __syncthreads();
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[((wave * NG + g) * 4 + r) * 64 + lane] = acc[g][r];
    __syncthreads();
    for (int v = threadIdx.x; v < NG * 4 * 64; v += kThreads) {
      const int g = v / 256, r = (v / 64) % 4, l = v % 64;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum += red[((w * NG + g) * 4 + r) * 64 + l];
      if (has_bias) sum += bf16_bits_to_f32(bias_bits);
      // D layout of the 16x16 MFMA: lane l holds rows 4*(l/16)+r of column l%16.
      const int m = 4 * (l >> 4) + r;
      const int n = row0 + 16 * g + (l & 15);
      if (m < M && n < N) {
        const int64_t o = (int64_t)m * N + n;
        if (OUT_BF16)
          reinterpret_cast<uint16_t *>(P.y)[o] = (uint16_t)(pack_bf16x2(sum, 0.0f) & 0xffffu);
        else
          reinterpret_cast<float *>(P.y)[o] = sum;
      }
    }
  }
}

// ---- x held in registers ----------------------------------------------------
// For K <= kXMaxK: a workgroup of 16 waves; wave w owns a fixed slice of the
// 128-code chunks of K (at most kXMaxCPW of them) and keeps x of that slice
// in registers, loaded once per problem. Persistent workgroups walk the work
// items (16 weight rows each) with two register sets of item loads in turn:
// the codes and scales of the next item are in flight while the current one
// is computed. Every load of an item goes through buffer resources whose
// range ends at the problem's last row, so rows past N read zeros, and the
// loads for a missing next item read nothing. The 16 partial tiles of an item
// are added in a fixed order through LDS (double-buffered, one barrier per
// item), so results are bitwise reproducible.
constexpr int kXWaves = 16;
constexpr int kXThreads = 64 * kXWaves;
constexpr int kXMaxCPW = 3;
constexpr int kXMaxK = kXWaves * kXMaxCPW * kChunk;  // 6144

// where an item's data lives and which chunks this wave computes
struct XItem {
  int pi;                    // problem
  int row0;                  // first weight row
  int c_begin, c_end;        // chunks of this wave
  int nch, kg_last;          // chunks of K; valid 32-code pieces of the last chunk
  __amdgpu_buffer_rsrc_t wrs, qrs, frs;
  int32_t g0;                // first scale group of the item (double quant)
};

template <bool DQ, int G>
__device__ __forceinline__ XItem x_item(const GemvArgs &args, int item, int wave) {
  XItem it;
  int pi = 0;
#pragma unroll 1
  while (pi + 1 < args.count && args.p[pi + 1].item_begin <= item) ++pi;
  const GemvProblem &P = args.p[pi];
  const int N = P.N, K = P.K;
  it.pi = pi;
  it.row0 = (item - P.item_begin) * 16 * G;
  it.nch = (K + kChunk - 1) / kChunk;
  it.c_begin = (wave * it.nch) / kXWaves;
  it.c_end = ((wave + 1) * it.nch) / kXWaves;
  it.kg_last = (K - (it.nch - 1) * kChunk) >> 5;
  const int rows = item < args.total_items ? (N - it.row0 < 16 * G ? N - it.row0 : 16 * G) : 0;
  const int64_t e0 = (int64_t)it.row0 * K;  // first element of the item
  const int64_t b0 = e0 >> P.log2_bs;        // its first block (K is a multiple of bs)
  const int nblk = (rows * K) >> P.log2_bs;
  it.wrs = __builtin_amdgcn_make_buffer_rsrc((void *)(P.packed + e0 / 2), (short)0,
                                             (rows * K) >> 1, kBufferFlags);
  if (DQ) {
    it.qrs = __builtin_amdgcn_make_buffer_rsrc((void *)(P.absmax_q + b0), (short)0, nblk,
                                               kBufferFlags);
    it.g0 = (int32_t)(b0 >> P.log2_bs2);
    const int ngr = rows ? (int)(((b0 + nblk - 1) >> P.log2_bs2) - it.g0 + 1) : 0;
    it.frs = __builtin_amdgcn_make_buffer_rsrc((void *)(P.absmax_scale + it.g0), (short)0, 4 * ngr,
                                               kBufferFlags);
  } else {
    it.qrs = it.wrs;
    it.g0 = 0;
    it.frs = __builtin_amdgcn_make_buffer_rsrc((void *)(P.absmax + b0), (short)0, 4 * nblk,
                                               kBufferFlags);
  }
  return it;
}

template <int CPW, int G>
struct XLoads {
  uint4 pw[CPW][G];
  float sf[CPW][G];
  int32_t sq[CPW][G];
};

// codes and scale parts of this lane's pieces of an item (a piece past K,
// last chunk only, reads the chunk start instead; its weights are zeroed later)
template <int CPW, int G, bool DQ>
__device__ __forceinline__ XLoads<CPW, G> x_issue(const GemvArgs &args, const XItem &it, int nl,
                                                  int kg) {
  XLoads<CPW, G> L;
  const GemvProblem &P = args.p[it.pi];
  const int K = P.K;
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    int c = it.c_begin + i;
    if (c >= it.c_end) c = it.c_end > it.c_begin ? it.c_end - 1 : 0;
    const int kc = c * kChunk + ((c == it.nch - 1 && kg >= it.kg_last) ? 0 : 32 * kg);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int e = (16 * g + nl) * K + kc;  // element of the item
      L.pw[i][g] =
          __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(it.wrs, e >> 1, 0, 0));
      const int b = e >> P.log2_bs;  // block within the item
      if (DQ) {
        L.sq[i][g] = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(it.qrs, b, 0, 0);
        const int gr = (int)((((int64_t)it.row0 * K >> P.log2_bs) + b) >> P.log2_bs2) - it.g0;
        L.sf[i][g] =
            __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(it.frs, 4 * gr, 0, 0));
      } else {
        L.sq[i][g] = 1;
        L.sf[i][g] =
            __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(it.frs, 4 * b, 0, 0));
      }
    }
  }
  return L;
}

// x of this wave's slice: lane (m, kg) holds x[m][kc + 32 kg .. + 31] of each
// chunk as four 16-byte pieces (rows m >= M read zeros)
template <int CPW>
__device__ __forceinline__ void x_load_x(const GemvArgs &args, const XItem &it, int nl, int kg,
                                         uint4 (&xa)[CPW][4]) {
  const GemvProblem &P = args.p[it.pi];
  const int M = args.M, K = P.K;
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc((void *)P.x, (short)0, M * K * 2, kBufferFlags);
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    int c = it.c_begin + i;
    if (c >= it.c_end) c = it.c_end > it.c_begin ? it.c_end - 1 : 0;
    const int kc = c * kChunk + ((c == it.nch - 1 && kg >= it.kg_last) ? 0 : 32 * kg);
    const int xoff = nl < M ? (nl * K + kc) * 2 : kOutOfRange;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      xa[i][s] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(xres, (int)((uint32_t)xoff + 16u * s), 0, 0));
  }
}

template <int CPW, int G, bool DQ, bool OUT_BF16>
__device__ __forceinline__ void x_compute(const GemvArgs &args, const XItem &it,
                                          const XLoads<CPW, G> &L, const uint4 (&xa)[CPW][4],
                                          const char *tbl, uint32_t lane_base, int lane, int kg,
                                          int wave, float *red) {
  // the bias of the output this thread writes at the end (threads < 256 G),
  // fetched before the item's arithmetic so its latency is hidden
  const GemvProblem &P = args.p[it.pi];
  const bool has_bias = P.bias != nullptr;
  uint32_t bias_bits;
  {
    const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)P.bias, (short)0, has_bias ? 2 * P.N : 0, kBufferFlags);
    bias_bits = __builtin_amdgcn_raw_buffer_load_b16(
        brs, 2 * (it.row0 + 16 * ((int)threadIdx.x >> 8) + ((int)threadIdx.x & 15)), 0, 0);
  }
  f32x4 acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = it.c_begin + i;
    const bool ok = c < it.c_end && (c < it.nch - 1 || kg < it.kg_last);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float ap = DQ ? (float)L.sq[i][g] * L.sf[i][g] : L.sf[i][g];
      ap = ok ? ap : 0.0f;
      const uint32_t words[4] = {L.pw[i][g].x, L.pw[i][g].y, L.pw[i][g].z, L.pw[i][g].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 b = dequant8(words[s], ap, tbl, lane_base);
        bf16x8 a = __builtin_bit_cast(bf16x8, xa[i][s]);
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[g], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[((wave * G + g) * 4 + r) * 64 + lane] = acc[g][r];
  __syncthreads();
  // 256 G of the threads each add one output over the 16 waves, in wave order
  static_assert(256 * G <= kXThreads, "one output per thread");
  if (threadIdx.x < 256 * G) {
    const int g = threadIdx.x >> 8, r = (threadIdx.x >> 6) & 3, l = threadIdx.x & 63;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kXWaves; ++w) sum += red[((w * G + g) * 4 + r) * 64 + l];
    if (has_bias) sum += bf16_bits_to_f32(bias_bits);
    // D layout of the 16x16 MFMA: lane l holds rows 4*(l/16)+r of column l%16.
    const int m = 4 * (l >> 4) + r;
    const int n = it.row0 + 16 * g + (l & 15);
    if (m < args.M && n < P.N) {
      const int64_t o = (int64_t)m * P.N + n;
      if (OUT_BF16)
        reinterpret_cast<uint16_t *>(P.y)[o] = (uint16_t)(pack_bf16x2(sum, 0.0f) & 0xffffu);
      else
        reinterpret_cast<float *>(P.y)[o] = sum;
    }
  }
}

template <int CPW, int G, bool DQ, bool OUT_BF16>
__global__ __launch_bounds__(kXThreads) void gemv_xreg_kernel(GemvArgs args) {
  __shared__ __attribute__((aligned(16))) char lds[kTableBytes + 2 * kXWaves * G * 4 * 64 * 4];
  const char *tbl = lds;
  float *red0 = reinterpret_cast<float *>(lds + kTableBytes);
  float *red1 = red0 + kXWaves * G * 4 * 64;

  // pair table, entry e = (value[e >> 4], value[e & 15]) at 256 e + 8 copy
  for (int idx = threadIdx.x; idx < 256 * kCopies; idx += kXThreads) {
    const int e = idx >> 5;
    const f32x2 v = {args.value[e >> 4], args.value[e & 15]};
    *reinterpret_cast<f32x2 *>(lds + 256 * e + 8 * (idx & 31)) = v;
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nl = lane & 15;
  const int kg = lane >> 4;
  const uint32_t lane_base = 8u * (uint32_t)(lane & (kCopies - 1));
  const int step = gridDim.x;

  int item = blockIdx.x;
  if (item >= args.total_items) return;  // whole workgroup
  XItem ia = x_item<DQ, G>(args, item, wave);
  XLoads<CPW, G> la = x_issue<CPW, G, DQ>(args, ia, nl, kg);
  uint4 xa[CPW][4];
  int xp = ia.pi;
  x_load_x<CPW>(args, ia, nl, kg, xa);
  __syncthreads();  // table built
  for (;;) {
    // item + step into the second set (an item past the end loads nothing)
    XItem ib = x_item<DQ, G>(args, item + step, wave);
    XLoads<CPW, G> lb = x_issue<CPW, G, DQ>(args, ib, nl, kg);
    x_compute<CPW, G, DQ, OUT_BF16>(args, ia, la, xa, tbl, lane_base, lane, kg, wave, red0);
    item += step;
    if (item >= args.total_items) break;
    if (ib.pi != xp) {
      x_load_x<CPW>(args, ib, nl, kg, xa);
      xp = ib.pi;
    }
    ia = x_item<DQ, G>(args, item + step, wave);
    la = x_issue<CPW, G, DQ>(args, ia, nl, kg);
    x_compute<CPW, G, DQ, OUT_BF16>(args, ib, lb, xa, tbl, lane_base, lane, kg, wave, red1);
    item += step;
    if (item >= args.total_items) break;
    if (ia.pi != xp) {
      x_load_x<CPW>(args, ia, nl, kg, xa);
      xp = ia.pi;
    }
  }
}

template <int CPW, int G, bool DQ>
hipError_t launch_xreg(const GemvArgs &args, int grid, bool out_bf16, hipStream_t stream) {
  if (out_bf16)
    hipLaunchKernelGGL((gemv_xreg_kernel<CPW, G, DQ, true>), dim3(grid), dim3(kXThreads), 0,
                       stream, args);
  else
    hipLaunchKernelGGL((gemv_xreg_kernel<CPW, G, DQ, false>), dim3(grid), dim3(kXThreads), 0,
                       stream, args);
  return hipGetLastError();
}

template <int NG, int CPW, bool DQ>
hipError_t launch_cfg(const GemvArgs &args, int grid, bool out_bf16, hipStream_t stream) {
  if (out_bf16)
    hipLaunchKernelGGL((gemv_kernel<NG, CPW, DQ, true>), dim3(grid), dim3(kThreads), 0, stream,
                       args);
  else
    hipLaunchKernelGGL((gemv_kernel<NG, CPW, DQ, false>), dim3(grid), dim3(kThreads), 0, stream,
                       args);
  return hipGetLastError();
}

template <bool DQ>
hipError_t launch_dq(const GemvArgs &args, int ng, int cpw, int grid, bool out_bf16,
                     hipStream_t stream) {
  if (ng == 2) return launch_cfg<2, 2, DQ>(args, grid, out_bf16, stream);
  if (cpw == 2) return launch_cfg<1, 2, DQ>(args, grid, out_bf16, stream);
  return launch_cfg<1, 4, DQ>(args, grid, out_bf16, stream);
}

}  // namespace

int gemv_max_group() { return kMaxGroup; }

namespace {

// Products with 2 <= M <= 16 and K <= kXMaxK, one launch of the x-in-registers kernel.
hipError_t launch_xreg_group(int count, const GemvDesc *descs, int M, int quant_type,
                             bool double_quant, bool out_bf16, hipStream_t stream) {
  const CodeTables &t = code_tables(quant_type);
  int rows_total = 0, max_k = 0;
  for (int i = 0; i < count; ++i) {
    rows_total += descs[i].N;
    max_k = descs[i].K > max_k ? descs[i].K : max_k;
  }
  const int nch = (max_k + kChunk - 1) / kChunk;
  const int cpw = (nch + kXWaves - 1) / kXWaves;
  // 32-row items (two accumulators per wave) put twice the bytes in flight per
  // item and halve the barriers; taken for short slices (at most 2 chunks per
  // wave, registers permitting) while every CU still gets several items
  const int g = (cpw <= 2 && rows_total / 32 >= 4 * device_cu_count()) ? 2 : 1;
  GemvArgs args;
  args.count = 0;
  args.M = M;
  int items = 0;
  for (int i = 0; i < count; ++i) {
    const GemvDesc &d = descs[i];
    if (d.N == 0) continue;
    GemvProblem &p = args.p[args.count++];
    p.x = d.x;
    p.packed = d.packed;
    p.y = d.y;
    p.bias = d.bias;
    p.absmax = d.sc.absmax;
    p.absmax_q = d.sc.absmax_q;
    p.absmax_scale = d.sc.absmax_scale;
    p.N = d.N;
    p.K = d.K;
    p.log2_bs = __builtin_ctz((unsigned)d.blocksize);
    p.log2_bs2 = d.sc.log2_bs2;
    p.item_begin = items;
    items += (d.N + 16 * g - 1) / (16 * g);
  }
  if (args.count == 0) return hipSuccess;
  args.total_items = items;
  for (int i = 0; i < 16; ++i) args.value[i] = t.value[i];
  const int cap = device_cu_count();
  const int grid = items < cap ? items : cap;
  if (g == 2) {
    if (double_quant)
      return cpw <= 1 ? launch_xreg<1, 2, true>(args, grid, out_bf16, stream)
                      : launch_xreg<2, 2, true>(args, grid, out_bf16, stream);
    return cpw <= 1 ? launch_xreg<1, 2, false>(args, grid, out_bf16, stream)
                    : launch_xreg<2, 2, false>(args, grid, out_bf16, stream);
  }
  if (double_quant) {
    if (cpw <= 1) return launch_xreg<1, 1, true>(args, grid, out_bf16, stream);
    if (cpw == 2) return launch_xreg<2, 1, true>(args, grid, out_bf16, stream);
    return launch_xreg<3, 1, true>(args, grid, out_bf16, stream);
  }
  if (cpw <= 1) return launch_xreg<1, 1, false>(args, grid, out_bf16, stream);
  if (cpw == 2) return launch_xreg<2, 1, false>(args, grid, out_bf16, stream);
  return launch_xreg<3, 1, false>(args, grid, out_bf16, stream);
}

hipError_t launch_split_group(int count, const GemvDesc *descs, int M, int quant_type,
                              bool double_quant, bool out_bf16, hipStream_t stream) {
  const CodeTables &t = code_tables(quant_type);
  // 32-row items share each x fragment between two MFMAs, but only while
  // there are enough of them to give every workgroup slot one
  int rows_total = 0;
  for (int i = 0; i < count; ++i) rows_total += descs[i].N;
  const int ng = (M > 4 && rows_total / 32 >= 2 * device_cu_count()) ? 2 : 1;
  GemvArgs args;
  args.count = 0;
  args.M = M;
  int items = 0, max_k = 0;
  for (int i = 0; i < count; ++i) {
    const GemvDesc &d = descs[i];
    if (d.N == 0) continue;
    GemvProblem &p = args.p[args.count++];
    p.x = d.x;
    p.packed = d.packed;
    p.y = d.y;
    p.bias = d.bias;
    p.absmax = d.sc.absmax;
    p.absmax_q = d.sc.absmax_q;
    p.absmax_scale = d.sc.absmax_scale;
    p.N = d.N;
    p.K = d.K;
    p.log2_bs = __builtin_ctz((unsigned)d.blocksize);
    p.log2_bs2 = d.sc.log2_bs2;
    p.item_begin = items;
    items += (d.N + 16 * ng - 1) / (16 * ng);
    max_k = d.K > max_k ? d.K : max_k;
  }
  if (args.count == 0) return hipSuccess;
  args.total_items = items;
  for (int i = 0; i < 16; ++i) args.value[i] = t.value[i];
  const int per_wave = ((max_k + kChunk - 1) / kChunk + kWaves - 1) / kWaves;
  const int cpw = per_wave <= 2 ? 2 : 4;
  // Two workgroups fit per CU (LDS); more items than that are walked in turn.
  const int cap = 2 * device_cu_count();
  const int grid = items < cap ? items : cap;
  return double_quant ? launch_dq<true>(args, ng, cpw, grid, out_bf16, stream)
                      : launch_dq<false>(args, ng, cpw, grid, out_bf16, stream);
}

}  // namespace

// Each product runs on the kernel it would get when launched alone (its
// K decides), so a product's result never depends on what it is grouped
// with: 2 <= M <= 16 with K <= kXMaxK take the x-in-registers kernel, the
// rest (and M = 1 here) the K-split kernel.
hipError_t launch_gemv_grouped(int count, const GemvDesc *descs, int M, int quant_type,
                               bool double_quant, bool out_bf16, hipStream_t stream) {
  if (count == 0 || M == 0) return hipSuccess;
  if (count > kMaxGroup) return hipErrorInvalidValue;
  if (M < 2) return launch_split_group(count, descs, M, quant_type, double_quant, out_bf16, stream);
  GemvDesc xs[kMaxGroup], rest[kMaxGroup];
  int nx = 0, nr = 0;
  for (int i = 0; i < count; ++i) {
    if (descs[i].K <= kXMaxK) xs[nx++] = descs[i];
    else rest[nr++] = descs[i];
  }
  hipError_t e = hipSuccess;
  if (nx) e = launch_xreg_group(nx, xs, M, quant_type, double_quant, out_bf16, stream);
  if (e == hipSuccess && nr)
    e = launch_split_group(nr, rest, M, quant_type, double_quant, out_bf16, stream);
  return e;
}

}  // namespace nf4
