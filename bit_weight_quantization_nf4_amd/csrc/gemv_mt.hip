// gemv_mt.hip -- decode products y_i[M, N_i] = x_i[M, K] . cd(dequant(W_i))^T
// for 1 <= M <= 64 on gfx950 matrix cores, one or several independent
// problems (sharing M and K) per launch; cd is the rounding to the compute
// dtype (bf16 or fp16).
//
// [repo page ossradar.top bitsandbytes, release notes 0.50.0: 4-bit inference
//  at batch 2..64 uses a fused 4-bit dequantize + GEMM in place of dequantize
//  + F.linear, with nested (double) quantization and the bias fused in, the
//  kernel chosen at run time from the shape; usage page icman.com.cn/news/48546,
//  "Configuration": weights are dequantized to the compute dtype before the
//  product.]
//
// Design (HBM-bound below M ~ 64: every 4-bit weight is read once):
//  - work items are 16 NT weight rows of one problem; a persistent workgroup
//    of W waves (one per CU) takes items blockIdx.x, + gridDim.x, ... and its
//    waves split K into W fixed contiguous ranges of 128-code chunks, so every
//    output is summed in the same order whatever the grouping, NT or grid;
//  - v_mfma_f32_16x16x32 with x as the A operand (rows m >= M read zeros) and
//    the dequantized weights as B. Lane (n, kg) = (l % 16, l / 16) loads the 32
//    codes k0 + 32 kg .. + 31 of row n of a chunk (16 bytes) and feeds four
//    MFMAs, one per 8-code word; the x fragments are loaded with the same k
//    permutation, so the order of k inside a chunk does not matter;
//  - a "unit" is one chunk of the wave's range for the NT row tiles of an item:
//    its code words, block-scale parts and x fragments. Each wave walks its
//    units item after item through a ring of D register sets, issuing unit
//    u + D - 1 before computing unit u; the ring runs on across item ends, so
//    the loads of the next item are in flight while an item's partial sums
//    are combined. Every unit issues the same loads (past the wave's last unit,
//    or past K, the offsets are out of range and read zeros without a memory
//    access), so the compiler's waits count exactly one unit's loads;
//  - dequantization through the conflict-free LDS pair table (entry = fp32
//    code values of both nibbles of a code byte, 32 interleaved copies, the
//    address built by one v_perm_b32), times the block scale, rounded to the
//    compute dtype in pairs;
//  - at an item's end the W partial tiles meet in LDS and are added in wave
//    order, then the optional bias (compute dtype) is added in fp32 and the
//    result rounded to the output dtype and stored (row stride ldy).
#include <limits.h>

#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kChunk = 128;              // codes of one row per unit
constexpr int kCopies = 32;              // interleaved copies of the pair table
constexpr int kTableBytes = 256 * 256;   // 256 entries x 256-byte rows
constexpr int kMaxGroup = 16;
constexpr int kMaxSplit = 8;             // K ranges of a split product, at most
constexpr int kBufferFlags = 0x00020000;  // word 3 of a raw buffer resource (gfx9)
constexpr uint32_t kOOB = 0x80000000u;    // an offset past every buffer's range

struct MtProblem {
  const char *x;          // activations (compute dtype), row m at m * ldx_bytes
  const uint8_t *packed;
  char *y;                // output, row m at m * ldy_bytes
  const char *bias;       // [N] compute dtype, or null
  const float *absmax;    // absmax (no double quant) or absmax_scale
  const int8_t *absmax_q;
  const float *absmax_offset;
  int32_t N;
  int32_t item_begin;     // first work item of the problem
  int32_t log2_bs, log2_bs2;
  uint32_t ldx_bytes, ldy_bytes;
  uint32_t x_bytes, y_bytes;  // ranges of x and y
  // K range of the problem (register-resident kernel): chunks kc0 .. kc1 - 1,
  // and the blocks of a row it reads, jb .. jb + jn - 1
  int32_t kc0, kc1, jb, jn;
};

struct MtArgs {
  int32_t item_begin[kMaxGroup];  // first item of each problem; unused: INT_MAX
  MtProblem p[kMaxGroup];
  int32_t count, M, K, total_items;
  int32_t out_dtype;
  int32_t nchs;  // chunks of a K range (the waves' split), register-resident kernel
  int32_t kbs;   // staged blocks of a row's K range (the most over the problems)
  int32_t nt;    // row tiles per item
  float value[16];
};

// 8 codes of one packed word -> 4 packed pairs of the compute type, in k order
// (byte j holds element 2j in its high nibble and 2j + 1 in its low nibble).
template <int CT>
__device__ __forceinline__ uint4 dequant8(uint32_t word, float ap, const char *tbl,
                                          uint32_t lane_base) {
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // address bytes: [0] lane_base (8 * copy), [1] code byte j, [2..3] zero
    const uint32_t addr = __builtin_amdgcn_perm(word, lane_base, 0x0c0c0000u | ((4u + j) << 8));
    const f32x2 c = *reinterpret_cast<const f32x2 *>(tbl + addr);
    out[j] = pack2<CT>(c.x * ap, c.y * ap);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

template <int MT, int NT, int PER>
struct Unit {
  uint4 w[NT];        // 32 codes of row 16 t + n
  int32_t q[NT];      // int8 block code (double quant)
  float s[NT];        // absmax, or the group scale s2
  float mu[NT];       // group offset (mean-centred double quant)
  uint4 xa[MT][4];    // x[16 mt + n][k0 + 32 kg + 8 s .. + 7]
  uint32_t bias[PER]; // bias bits of the outputs this thread stores at the item's end
};

template <int W, int MT, int NT, int DQ, int CT>
__global__ __launch_bounds__(64 * W) void gemv_mt_kernel(MtArgs args) {
  constexpr int D = 2;  // units in the ring
  __shared__ __attribute__((aligned(16))) char tbl[kTableBytes];
  __shared__ __attribute__((aligned(16))) float red[W * NT * MT * 4 * 64];
  __shared__ float vals[16];

  if (threadIdx.x < 16) vals[threadIdx.x] = args.value[threadIdx.x];
  __syncthreads();
  // pair table, entry e = (value[e >> 4], value[e & 15]) at 256 e + 8 copy;
  // consecutive threads write consecutive copies
  for (int idx = threadIdx.x; idx < 256 * kCopies; idx += 64 * W) {
    const int e = idx >> 5;
    const f32x2 v = {vals[e >> 4], vals[e & 15]};
    *reinterpret_cast<f32x2 *>(tbl + 256 * e + 8 * (idx & 31)) = v;
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int n = lane & 15, kg = lane >> 4;
  const uint32_t lane_base = 8u * (uint32_t)(lane & (kCopies - 1));
  const int M = args.M, K = args.K;
  const int nch = (K + kChunk - 1) / kChunk;
  const int c0 = (wave * nch) / W, c1 = ((wave + 1) * nch) / W;
  const int items = args.total_items;
  const int I = (int)blockIdx.x < items ? (items - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const uint32_t row_bytes = (uint32_t)K >> 1;

  int ib[kMaxGroup];
#pragma unroll
  for (int k = 0; k < kMaxGroup; ++k) ib[k] = args.item_begin[k];
  // problem of an item: a short compare chain over the first items (scalar;
  // the array is never indexed by a computed value, which would move it to
  // vector registers)
  auto problem_of = [&](int item) {
    int p = 0;
#pragma unroll
    for (int k = 1; k < kMaxGroup; ++k) p = ib[k] <= item ? k : p;
    return p;
  };

  // outputs of the item's end: thread t stores output o = t + 64 W j
  constexpr int kOuts = NT * MT * 256;
  constexpr int kPer = (kOuts + 64 * W - 1) / (64 * W);

  // Loads of unit (item ordinal i of this workgroup, chunk c). Past the
  // workgroup's items every offset is out of range. Every unit also fetches
  // the bias of the outputs this thread stores at an item's end (used after
  // the item's last unit): a load issued there would be the newest in flight,
  // and waiting for it would drain the ring.
  auto issue = [&](int i, int c) {
    Unit<MT, NT, kPer> u;
    const bool valid = i < I;
    const int item = (int)blockIdx.x + (valid ? i : 0) * (int)gridDim.x;
    const int p = problem_of(item);
    const MtProblem &P = args.p[p];
    const int row0 = (item - P.item_begin) * 16 * NT;
    const int rows = P.N - row0 < 16 * NT ? P.N - row0 : 16 * NT;
    const int k0 = c * kChunk + 32 * kg;
    const bool kok = valid && k0 < K;
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(P.packed + (int64_t)row0 * row_bytes), (short)0, (int)((uint32_t)rows * row_bytes),
        kBufferFlags);
    // the item's first block, and its group split into a group base and the
    // block's place in that group (64-bit safe)
    const uint64_t blk0 = ((uint64_t)row0 * (uint64_t)K) >> P.log2_bs;
    const uint32_t nblk = ((uint32_t)rows * (uint32_t)K) >> P.log2_bs;
    const uint64_t g0 = DQ ? blk0 >> P.log2_bs2 : 0;
    const uint32_t blk_in = DQ ? (uint32_t)(blk0 & ((1ull << P.log2_bs2) - 1)) : 0;
    const uint32_t ngr = DQ ? (blk_in + nblk + (1u << P.log2_bs2) - 1) >> P.log2_bs2 : 0;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(P.absmax + (DQ ? g0 : blk0)), (short)0, (int)(4u * (DQ ? ngr : nblk)),
        kBufferFlags);
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(DQ ? (const void *)(P.absmax_q + blk0) : (const void *)P.absmax), (short)0,
        (int)(DQ ? nblk : 0u), kBufferFlags);
    const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(DQ == kDqCentred ? P.absmax_offset + g0 : P.absmax), (short)0,
        (int)(DQ == kDqCentred ? 4u * ngr : 0u), kBufferFlags);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t r = (uint32_t)(16 * t + n);
      u.w[t] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     wrs, (int)(kok ? r * row_bytes + ((uint32_t)k0 >> 1) : kOOB), 0, 0));
      const uint32_t b = (r * (uint32_t)K + (uint32_t)k0) >> P.log2_bs;  // block in the item
      if (DQ == kDqNone) {
        u.q[t] = 1;
        u.mu[t] = 0.0f;
        u.s[t] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(srs, (int)(kok ? 4u * b : kOOB), 0, 0));
      } else {
        const uint32_t g = (blk_in + b) >> P.log2_bs2;
        u.q[t] = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(qrs, (int)(kok ? b : kOOB), 0, 0);
        u.s[t] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(srs, (int)(kok ? 4u * g : kOOB), 0, 0));
        if (DQ == kDqCentred)
          u.mu[t] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(mrs, (int)(kok ? 4u * g : kOOB), 0, 0));
        else
          u.mu[t] = 0.0f;
      }
    }
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)P.x, (short)0, (int)P.x_bytes, kBufferFlags);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = 16 * mt + n;
      const uint32_t off = (kok && m < M) ? (uint32_t)m * P.ldx_bytes + 2u * (uint32_t)k0 : kOOB;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        u.xa[mt][s] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)(off + 16u * s), 0, 0));
    }
    const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)P.bias, (short)0, P.bias != nullptr ? (int)(2u * (uint32_t)P.N) : 0, kBufferFlags);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int o = (int)threadIdx.x + 64 * W * j;
      const int row = row0 + 16 * ((o >> 8) / MT) + (o & 15);
      u.bias[j] = __builtin_amdgcn_raw_buffer_load_b16(brs, (int)(2u * (uint32_t)row), 0, 0);
    }
    return u;
  };

  f32x4 acc[NT][MT];
  auto zero = [&]() {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  auto compute = [&](const Unit<MT, NT, kPer> &u) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float ap = scale_from<DQ>(u.q[t], u.s[t], u.mu[t]);
      const uint32_t wd[4] = {u.w[t].x, u.w[t].y, u.w[t].z, u.w[t].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 b = dequant8<CT>(wd[s], ap, tbl, lane_base);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = mfma16x16x32<CT>(u.xa[mt][s], b, acc[t][mt]);
      }
    }
  };

  // The end of item ordinal i: partial tiles through LDS, added in wave order
  // by the threads that own the outputs, bias, rounding and store.
  auto finish = [&](int i, const uint32_t (&bias_bits)[kPer]) {
    const int item = (int)blockIdx.x + i * (int)gridDim.x;
    const int p = problem_of(item);
    const MtProblem &P = args.p[p];
    const int row0 = (item - P.item_begin) * 16 * NT;
    const bool has_bias = P.bias != nullptr;
    __syncthreads();  // the previous item's sums have been read
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[(((wave * NT + t) * MT + mt) * 4 + r) * 64 + lane] = acc[t][mt][r];
    __syncthreads();
    const int ob = args.out_dtype == kFP32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)P.y, (short)0, (int)P.y_bytes, kBufferFlags);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int o = (int)threadIdx.x + 64 * W * j;
      if (kOuts % (64 * W) != 0 && o >= kOuts) break;
      const int l = o & 63, r = (o >> 6) & 3, mt = (o >> 8) % MT, t = (o >> 8) / MT;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) sum += red[(((w * NT + t) * MT + mt) * 4 + r) * 64 + l];
      if (has_bias) sum += widen16<CT>(bias_bits[j]);
      // D layout of the 16x16 MFMA: lane l holds rows 4 (l / 16) + r of column l % 16
      const int m = 16 * mt + 4 * (l >> 4) + r;
      const int row = row0 + 16 * t + (l & 15);
      const uint32_t off = (m < M && row < P.N)
                               ? (uint32_t)m * P.ldy_bytes + (uint32_t)row * (uint32_t)ob
                               : kOOB;
      if (args.out_dtype == kFP32)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sum), yrs, (int)off, 0, 0);
      else if (args.out_dtype == kFP16)
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)out_bits<kFP16>(sum), yrs, (int)off, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)out_bits<kBF16>(sum), yrs, (int)off, 0, 0);
    }
  };

  zero();
  __syncthreads();  // table built
  if (c1 == c0) {
    // no chunks for this wave (K below W chunks): zero partials, same barriers
    // (a unit of chunk 0 fetches the bias; its codes are not used)
    for (int i = 0; i < I; ++i) {
      const Unit<MT, NT, kPer> u = issue(i, 0);
      finish(i, u.bias);
    }
    return;
  }
  // issue pointer (item ordinal, chunk) runs D - 1 units ahead of the compute
  // pointer
  int is_i = 0, is_c = c0;
  auto advance = [&]() {
    if (++is_c == c1) {
      is_c = c0;
      ++is_i;
    }
  };
  Unit<MT, NT, kPer> ring[D];
#pragma unroll
  for (int j = 0; j < D - 1; ++j) {
    ring[j] = issue(is_i, is_c);
    advance();
  }
  const int U = I * (c1 - c0);
  int cu_i = 0, cu_c = c0;
  for (int u0 = 0; u0 < U; u0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      ring[(j + D - 1) % D] = issue(is_i, is_c);
      advance();
      if (u0 + j < U) {
        compute(ring[j]);
        if (++cu_c == c1) {
          finish(cu_i, ring[j].bias);
          zero();
          cu_c = c0;
          ++cu_i;
        }
      }
    }
  }
}

// ---- x held in registers (M <= 64; a K range of at most 16 * 128 * CMAX) ---
// The same K split over 16 waves, but each wave keeps x of its chunk range in
// registers (MT row tiles of 16 activation rows), loaded when the workgroup
// reaches a problem with other activations or another K range; a unit is then
// a whole item of the wave (its CMAX chunks, the ones past its range reading
// zeros), and the ring runs over items. The workgroups take contiguous item
// ranges, so a workgroup changes problems only at the few boundaries inside
// its range. Without a K split every output is summed in the same order as by
// the streaming kernel, so both give identical results.
//
// K split. x of a long row does not fit the registers of one CU (16 rows of
// K = 11008 are 352 KB; 64 rows of K = 4096, 512 KB). A problem then covers
// one K range [kc0, kc1) of a product (chunks kc0 .. kc1 - 1, the launch's
// nchs chunks at most) and writes its fp32 partial sums to a workspace; a
// second kernel adds the ranges of each output in range order, then the
// bias, and rounds. Every range of a product has the same nchs-chunk split
// over the waves, so the result depends only on M and K.
//
// The waves of a workgroup move through the items together (a barrier per
// item): each wave reads only its 128-code slices of a row, so the item's
// rows are fetched as whole DRAM pages only while all 16 waves ask for them
// at about the same time. Within an item, the code words of the item D - 1
// ahead are issued chunk by chunk between this item's chunks, so address
// processing overlaps arithmetic, and a wave lowers its priority as it gets
// through the item, so the four waves sharing a SIMD finish together rather
// than oldest-first.
//
// Block scales are staged: one item ahead, the whole workgroup loads the
// item's block codes (and group scales) of its K range row by row -- a wave
// reads 64 consecutive blocks of a row, so every load is one or two cache
// lines, and each block is read once per workgroup instead of once per wave
// and piece -- forms a' = scale_from(q, s2, mu) once per block and writes it
// to an LDS buffer (two buffers, alternating by item); a lane then reads the
// scale of each of its 32-code pieces from LDS. Rows of the staged item are
// RS floats apart with RS = 4 (mod 64), so the 16 rows x (up to 4) blocks a
// wave reads at once fall in distinct banks.
// BPC: blocks per 128-code chunk the staging is sized for (4: blocksize 32; 2:
// blocksize 64 and up -- a range of blocksize >= 256 may start inside a block,
// which its extra block fits in).
template <int W, int NT, int CMAX, int BPC>
struct XStage {
  static constexpr int kRows = 16 * NT;
  static constexpr int kTpr = 64 * W / kRows;       // staging threads per row
  static constexpr int kMaxBlocks = W * CMAX * BPC; // blocks of a row's K range
  static constexpr int kMaxPitch = kMaxBlocks + ((4 - kMaxBlocks) & 63);
  static constexpr int kSlots = (kMaxBlocks + kTpr - 1) / kTpr;
  static constexpr int kBufFloats = kRows * kMaxPitch;
};

template <int NT, int CMAX, int SLOTS, int PER>
struct XUnit {
  uint4 w[CMAX][NT];
  int32_t q[SLOTS];     // staged blocks: int8 block code (double quant)
  float s[SLOTS];       // absmax, or the group scale s2
  float mu[SLOTS];      // group offset (mean-centred double quant)
  uint32_t bias[PER];
  int32_t p;            // problem (uniform)
};

// s_setprio with a value known after unrolling
__device__ __forceinline__ void set_priority(int v) {
  if (v >= 3) __builtin_amdgcn_s_setprio(3);
  else if (v == 2) __builtin_amdgcn_s_setprio(2);
  else if (v == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

template <int W, int NT, int CMAX, int D, int DQ, int CT, int MT, int BPC>
__global__ __launch_bounds__(64 * W) void gemv_mtx_kernel(MtArgs args) {
  using SD = XStage<W, NT, CMAX, BPC>;
  // partial-sum buffers: two (one barrier per item) where LDS allows
  constexpr int kRedFloats = W * NT * MT * 4 * 64;
  constexpr int RB = kTableBytes + 4 * (2 * kRedFloats + 2 * SD::kBufFloats) <= 160 * 1024 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) char tbl[kTableBytes];
  __shared__ __attribute__((aligned(16))) float red[RB * kRedFloats];
  __shared__ __attribute__((aligned(16))) float stage[2 * SD::kBufFloats];
  __shared__ float vals[16];

  if (threadIdx.x < 16) vals[threadIdx.x] = args.value[threadIdx.x];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int n = lane & 15, kg = lane >> 4;
  const uint32_t lane_base = 8u * (uint32_t)(lane & (kCopies - 1));
  const int M = args.M, K = args.K;
  // this wave's chunks of a problem's K range: kc0 + w0 .. kc0 + w1 - 1
  // (and below the range's end kc1)
  const int nchs = args.nchs;
  const int w0 = (wave * nchs) / W, w1 = ((wave + 1) * nchs) / W;
  // this workgroup's items: a contiguous range
  const int items = args.total_items;
  const int ibeg = (int)(((int64_t)blockIdx.x * items) / gridDim.x);
  const int iend = (int)(((int64_t)(blockIdx.x + 1) * items) / gridDim.x);
  const int I = iend - ibeg;
  const uint32_t row_bytes = (uint32_t)K >> 1;
  constexpr int kOuts = NT * MT * 256;
  constexpr int kPer = (kOuts + 64 * W - 1) / (64 * W);
  // every problem of the launch has the same blocksize
  const int log2_bs = args.p[0].log2_bs;
  const int KB = K >> log2_bs;                  // blocks of a row
  const int KBS = args.kbs;                     // staged blocks of a row's K range
  const int RS = KBS + ((4 - KBS) & 63);        // staged row pitch (floats)
  // staging: thread -> (row sr of the item, blocks sj + kTpr v)
  const int sr = (int)threadIdx.x / SD::kTpr, sj = (int)threadIdx.x % SD::kTpr;

  int ib[kMaxGroup];
#pragma unroll
  for (int k = 0; k < kMaxGroup; ++k) ib[k] = args.item_begin[k];
  auto problem_of = [&](int item) {
    int p = 0;
#pragma unroll
    for (int k = 1; k < kMaxGroup; ++k) p = ib[k] <= item ? k : p;
    return p;
  };

  // this lane's staged scale of each piece (chunk cc of the wave's range;
  // row tile t is 64 RS bytes on); pieces past the wave's range, the
  // problem's range or K take scale 0 (their codes and x read zeros). Set for
  // the problem whose x is held.
  uint32_t saddr[CMAX];
  bool sok[CMAX];
  int c0 = 0;
  auto set_range = [&](const MtProblem &P) {
    c0 = P.kc0 + w0;
    const int c1 = P.kc0 + w1 < P.kc1 ? P.kc0 + w1 : P.kc1;
#pragma unroll
    for (int cc = 0; cc < CMAX; ++cc) {
      const int k0 = (c0 + cc) * kChunk + 32 * kg;
      sok[cc] = c0 + cc < c1 && k0 < K;
      const int j = sok[cc] ? (k0 >> log2_bs) - P.jb : 0;
      saddr[cc] = 4u * (uint32_t)(n * RS + j);
    }
  };

  using U = XUnit<NT, CMAX, SD::kSlots, kPer>;
  // where item ordinal i's loads come from
  struct Src {
    __amdgpu_buffer_rsrc_t wrs;
    int c0, c1;  // the wave's chunks of the item (scalar)
    bool valid;
  };
  // Loads of item ordinal i except its code words: the staged scales (first,
  // so that the wait before they are written to LDS leaves the code words in
  // flight) and the bias of the outputs this thread stores at the item's end.
  // Past the workgroup's items every offset is out of range.
  auto issue_head = [&](int i, U &u) {
    const bool valid = i < I;
    const int item = ibeg + (valid ? i : 0);
    const int p = problem_of(item);
    u.p = p;
    const MtProblem &P = args.p[p];
    const int row0 = (item - P.item_begin) * 16 * NT;
    const int rows = P.N - row0 < 16 * NT ? P.N - row0 : 16 * NT;
    const uint64_t blk0 = ((uint64_t)row0 * (uint64_t)K) >> log2_bs;
    const uint32_t nblk = (uint32_t)rows * (uint32_t)KB;
    const uint64_t g0 = DQ ? blk0 >> P.log2_bs2 : 0;
    const uint32_t blk_in = DQ ? (uint32_t)(blk0 & ((1ull << P.log2_bs2) - 1)) : 0;
    const uint32_t ngr = DQ ? (blk_in + nblk + (1u << P.log2_bs2) - 1) >> P.log2_bs2 : 0;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(P.absmax + (DQ ? g0 : blk0)), (short)0,
        valid ? (int)(4u * (DQ ? ngr : nblk)) : 0, kBufferFlags);
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(DQ ? (const void *)(P.absmax_q + blk0) : (const void *)P.absmax), (short)0,
        (int)(DQ && valid ? nblk : 0u), kBufferFlags);
    const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(DQ == kDqCentred ? P.absmax_offset + g0 : P.absmax), (short)0,
        (int)(DQ == kDqCentred && valid ? 4u * ngr : 0u), kBufferFlags);
    // (every slot's loads are issued, unused ones out of range: a load under a
    // branch would be waited for where the branches join)
#pragma unroll
    for (int v = 0; v < SD::kSlots; ++v) {
      const int j = sj + SD::kTpr * v;
      const uint32_t b = (uint32_t)(sr * KB + P.jb + j);  // block in the item
      const bool ok = j < P.jn;
      u.q[v] = 1;
      u.mu[v] = 0.0f;
      if (DQ == kDqNone) {
        u.s[v] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(srs, (int)(ok ? 4u * b : kOOB), 0, 0));
      } else {
        const uint32_t g = (blk_in + b) >> P.log2_bs2;
        u.q[v] = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(qrs, (int)(ok ? b : kOOB), 0, 0);
        u.s[v] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(srs, (int)(ok ? 4u * g : kOOB), 0, 0));
        if (DQ == kDqCentred)
          u.mu[v] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(mrs, (int)(ok ? 4u * g : kOOB), 0, 0));
      }
    }
    const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)P.bias, (short)0, P.bias != nullptr ? (int)(2u * (uint32_t)P.N) : 0, kBufferFlags);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int o = (int)threadIdx.x + 64 * W * j;
      const int row = row0 + 16 * ((o >> 8) / MT) + (o & 15);
      u.bias[j] = __builtin_amdgcn_raw_buffer_load_b16(brs, (int)(2u * (uint32_t)row), 0, 0);
    }
    Src src;
    src.valid = valid;
    src.c0 = P.kc0 + w0;
    src.c1 = P.kc0 + w1 < P.kc1 ? P.kc0 + w1 : P.kc1;
    src.wrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(P.packed + (int64_t)row0 * row_bytes), (short)0,
        (int)((uint32_t)rows * row_bytes), kBufferFlags);
    return src;
  };
  // the code words of chunk cc of the item
  auto issue_chunk = [&](const Src &src, int cc, U &u) {
    const int k0 = (src.c0 + cc) * kChunk + 32 * kg;
    const bool kok = src.valid && src.c0 + cc < src.c1 && k0 < K;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t r = (uint32_t)(16 * t + n);
      u.w[cc][t] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     src.wrs, (int)(kok ? r * row_bytes + ((uint32_t)k0 >> 1) : kOOB), 0, 0));
    }
  };

  // a' of the unit's staged blocks into stage buffer `buf` (rows past the
  // problem's N, and blocks past its K range, read zero codes and are never
  // used)
  auto write_stage = [&](const U &u, int buf) {
    float *sb = stage + buf * SD::kBufFloats + sr * RS;
#pragma unroll
    for (int v = 0; v < SD::kSlots; ++v) {
      const int j = sj + SD::kTpr * v;
      if (j < KBS) sb[j] = scale_from<DQ>(u.q[v], u.s[v], u.mu[v]);
    }
  };

  // x of the wave's chunks for problem p, MT row tiles (rows m >= M and
  // pieces past K or past the wave's range read zeros); set_range(p) first
  uint4 xr[CMAX][MT][4];
  auto load_x = [&](int p) {
    const MtProblem &P = args.p[p];
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)P.x, (short)0, (int)P.x_bytes, kBufferFlags);
#pragma unroll
    for (int cc = 0; cc < CMAX; ++cc) {
      const int k0 = (c0 + cc) * kChunk + 32 * kg;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + n;
        const bool ok = sok[cc] && m < M;
        const uint32_t off = ok ? (uint32_t)m * P.ldx_bytes + 2u * (uint32_t)k0 : kOOB;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          xr[cc][mt][s] = __builtin_bit_cast(
              uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)(off + 16u * s), 0, 0));
      }
    }
  };

  // Wait for x where it was loaded: past a branch (or into the loop) the
  // compiler would otherwise count x among the newest loads and make every
  // later wait for x also wait for the items in flight.
  auto touch_x = [&]() {
#pragma unroll
    for (int cc = 0; cc < CMAX; ++cc)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          asm volatile("" ::"v"(xr[cc][mt][s].x), "v"(xr[cc][mt][s].y), "v"(xr[cc][mt][s].z),
                       "v"(xr[cc][mt][s].w));
  };

  f32x4 acc[NT][MT];
  // chunk cc of a unit (stage buffer `buf`)
  // The table reads of LA 8-code words go out before their arithmetic, and
  // their LA operands are formed before their MFMAs, so the table latency is
  // paid once per LA words and the matrix core gets LA * MT multiply-adds back
  // to back. LA = 4 (the whole piece) in the 8-wave layout; 2 where 128
  // registers per wave would not hold four (1 with two row tiles of x).
  auto compute_chunk = [&](const U &u, int cc, int buf) {
    constexpr int LA = W == 8 ? 4 : (MT == 1 ? 2 : 1);
    const char *sb = reinterpret_cast<const char *>(stage) + buf * (4 * SD::kBufFloats);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float ap = *reinterpret_cast<const float *>(sb + saddr[cc] + 64 * RS * t);
      ap = sok[cc] ? ap : 0.0f;
      const uint32_t wd[4] = {u.w[cc][t].x, u.w[cc][t].y, u.w[cc][t].z, u.w[cc][t].w};
#pragma unroll
      for (int s0 = 0; s0 < 4; s0 += LA) {
        f32x2 cv[LA][4];
#pragma unroll
        for (int s = 0; s < LA; ++s)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t addr =
                __builtin_amdgcn_perm(wd[s0 + s], lane_base, 0x0c0c0000u | ((4u + j) << 8));
            cv[s][j] = *reinterpret_cast<const f32x2 *>(tbl + addr);
          }
        uint4 b[LA];
#pragma unroll
        for (int s = 0; s < LA; ++s)
          b[s] = make_uint4(pack2<CT>(cv[s][0].x * ap, cv[s][0].y * ap),
                            pack2<CT>(cv[s][1].x * ap, cv[s][1].y * ap),
                            pack2<CT>(cv[s][2].x * ap, cv[s][2].y * ap),
                            pack2<CT>(cv[s][3].x * ap, cv[s][3].y * ap));
#pragma unroll
        for (int s = 0; s < LA; ++s)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[t][mt] = mfma16x16x32<CT>(xr[cc][mt][s0 + s], b[s], acc[t][mt]);
      }
    }
  };

  // With two partial buffers, item ordinal i uses buffer i & 1: its last
  // reader, item i - 2, was done by every wave before the barrier of item i - 1.
  auto finish = [&](int i, const U &u) {
    const int item = ibeg + i;
    const MtProblem &P = args.p[u.p];
    const int row0 = (item - P.item_begin) * 16 * NT;
    const bool has_bias = P.bias != nullptr;
    float *rb = red + (RB == 2 ? (i & 1) * kRedFloats : 0);
    if (RB == 1) __syncthreads();  // the previous item's sums have been read
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          rb[(((wave * NT + t) * MT + mt) * 4 + r) * 64 + lane] = acc[t][mt][r];
    __syncthreads();
    const int ob = args.out_dtype == kFP32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)P.y, (short)0, (int)P.y_bytes, kBufferFlags);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int o = (int)threadIdx.x + 64 * W * j;
      if (kOuts % (64 * W) != 0 && o >= kOuts) break;
      const int l = o & 63, r = (o >> 6) & 3, mt = (o >> 8) % MT, t = (o >> 8) / MT;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) sum += rb[(((w * NT + t) * MT + mt) * 4 + r) * 64 + l];
      if (has_bias) sum += widen16<CT>(u.bias[j]);
      // D layout of the 16x16 MFMA: lane l holds rows 4 (l / 16) + r of column l % 16
      const int m = 16 * mt + 4 * (l >> 4) + r;
      const int row = row0 + 16 * t + (l & 15);
      const uint32_t off = (m < M && row < P.N)
                               ? (uint32_t)m * P.ldy_bytes + (uint32_t)row * (uint32_t)ob
                               : kOOB;
      if (args.out_dtype == kFP32)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sum), yrs, (int)off, 0, 0);
      else if (args.out_dtype == kFP16)
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)out_bits<kFP16>(sum), yrs, (int)off, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)out_bits<kBF16>(sum), yrs, (int)off, 0, 0);
    }
  };

  if (I <= 0) return;  // (whole workgroup; never taken: the grid is at most the item count)
  // Ring of D item units, issued D - 1 items ahead; item ordinal i uses stage
  // buffer i & 1. The stage of item i + 1 is written after item i is
  // computed: every wave has left item i - 1 (the buffer's last reader) at
  // the barrier of its end, and the barrier of item i's end publishes the
  // stage before item i + 1 is computed. Before issuing, the x of the unit
  // about to be computed is loaded if its activations or K range differ from
  // the ones held. The first units are issued before the pair table is
  // built, so the table's construction hides their latency.
  // The activations are loaded first, then the first items: loads complete
  // in order, so the wait for x is then not also a wait for the first items'
  // codes (on one [11008, 4096] product at M = 4 that order took 13.7 ->
  // 13.0 us, on a 7B layer at M = 16 39.3 -> 38.5 us).
  U ring[D];
  const int p_first = problem_of(ibeg);
  set_range(args.p[p_first]);
  load_x(p_first);
#pragma unroll
  for (int k = 0; k < D - 1; ++k) {
    const Src src = issue_head(k, ring[k]);
#pragma unroll
    for (int cc = 0; cc < CMAX; ++cc) issue_chunk(src, cc, ring[k]);
  }
  const char *x_held = args.p[p_first].x;
  uint32_t x_ld = args.p[p_first].ldx_bytes;
  int kc_held = args.p[p_first].kc0;
  __syncthreads();  // code values in LDS
  for (int idx = threadIdx.x; idx < 256 * kCopies; idx += 64 * W) {
    const int e = idx >> 5;
    const f32x2 v = {vals[e >> 4], vals[e & 15]};
    *reinterpret_cast<f32x2 *>(tbl + 256 * e + 8 * (idx & 31)) = v;
  }
  touch_x();
  write_stage(ring[0], 0);
  __syncthreads();  // table and the first stage built
  for (int i0 = 0; i0 < I; i0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int i = i0 + j;
      const bool live = i < I;
      if (live) {
        const MtProblem &P = args.p[ring[j].p];
        if (P.x != x_held || P.ldx_bytes != x_ld || P.kc0 != kc_held) {
          set_range(P);
          load_x(ring[j].p);
          touch_x();
          x_held = P.x;
          x_ld = P.ldx_bytes;
          kc_held = P.kc0;
        }
      }
      // (a unit past the workgroup's items is computed too, from zero codes,
      // and never stored: a load under a branch would be waited for where
      // the branches join)
      U &nu = ring[(j + D - 1) % D];
      const Src src = issue_head(i + D - 1, nu);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < CMAX; ++cc) {
        set_priority(CMAX - 1 - cc);
        compute_chunk(ring[j], cc, i & 1);
        issue_chunk(src, cc, nu);
      }
      __builtin_amdgcn_s_setprio(0);
      if (i + 1 < I) write_stage(ring[(j + 1) % D], (i + 1) & 1);
      if (live) finish(i, ring[j]);
    }
  }
}

// The split-K sums: y_i[m, n] = out(sum over r < S of part_i[r][m][n], in
// range order, + bias_i[n]) for the products of a split launch. part_i is
// [S][M][N] fp32, contiguous. A thread takes four consecutive n of one row.
struct SplitReduceProblem {
  const float *part;
  char *y;               // row m at m * ldy_bytes
  const char *bias;      // [N] compute dtype, or null
  int32_t N;
  int32_t S;             // K ranges of the problem (1 .. kMaxSplit)
  uint32_t ldy_bytes;
  int32_t block_begin;   // first workgroup of the problem
};

struct SplitReduceArgs {
  int32_t block_begin[kMaxGroup];  // unused: INT_MAX
  SplitReduceProblem p[kMaxGroup];
  int32_t M, out_dtype;
};

constexpr int kReduceThreads = 256;

template <int CT>
__global__ __launch_bounds__(kReduceThreads) void gemv_split_reduce_kernel(SplitReduceArgs args) {
  int p = 0;
#pragma unroll
  for (int k = 1; k < kMaxGroup; ++k) p = args.block_begin[k] <= (int)blockIdx.x ? k : p;
  const SplitReduceProblem &P = args.p[p];
  const int N = P.N, M = args.M, S = P.S;
  const int n4 = (N + 3) >> 2;  // quads of a row
  const int64_t q = (int64_t)((int)blockIdx.x - P.block_begin) * kReduceThreads + threadIdx.x;
  if (q >= (int64_t)M * n4) return;
  const int m = (int)(q / n4), n = 4 * (int)(q % n4);
  const uint32_t plane = (uint32_t)M * (uint32_t)N;  // floats of one range
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.part, (short)0, (int)(4u * plane * (uint32_t)S), kBufferFlags);
  // every range's four values are loaded before any is added (one memory
  // round trip); ranges past S read zeros and are not added
  const uint32_t e0 = (uint32_t)m * (uint32_t)N + (uint32_t)n;
  float v[kMaxSplit][4];
  if ((N & 3) == 0) {  // whole quads, 16-byte aligned
#pragma unroll
    for (int r = 0; r < kMaxSplit; ++r) {
      const uint32_t off = r < S ? 4u * (e0 + (uint32_t)r * plane) : kOOB;
      const f32x4 t = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(prs, (int)off, 0, 0));
#pragma unroll
      for (int j = 0; j < 4; ++j) v[r][j] = t[j];
    }
  } else {
#pragma unroll
    for (int r = 0; r < kMaxSplit; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t off = r < S && n + j < N ? 4u * (e0 + j + (uint32_t)r * plane) : kOOB;
        v[r][j] = __builtin_bit_cast(float,
                                     __builtin_amdgcn_raw_buffer_load_b32(prs, (int)off, 0, 0));
      }
  }
  float sum[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sum[j] = v[0][j];
#pragma unroll
  for (int r = 1; r < kMaxSplit; ++r)
    if (r < S)
#pragma unroll
      for (int j = 0; j < 4; ++j) sum[j] += v[r][j];
  const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.bias, (short)0, P.bias != nullptr ? (int)(2u * (uint32_t)N) : 0, kBufferFlags);
  const int ob = args.out_dtype == kFP32 ? 4 : 2;
  const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.y, (short)0, (int)((uint32_t)(M - 1) * P.ldy_bytes + (uint32_t)N * ob),
      kBufferFlags);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float v = sum[j];
    if (P.bias != nullptr)
      v += widen16<CT>(__builtin_amdgcn_raw_buffer_load_b16(brs, (int)(2u * (uint32_t)(n + j)), 0, 0));
    const uint32_t off =
        n + j < N ? (uint32_t)m * P.ldy_bytes + (uint32_t)(n + j) * (uint32_t)ob : kOOB;
    if (args.out_dtype == kFP32)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), yrs, (int)off, 0, 0);
    else if (args.out_dtype == kFP16)
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)out_bits<kFP16>(v), yrs, (int)off, 0, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)out_bits<kBF16>(v), yrs, (int)off, 0, 0);
  }
}

template <int W, int MT, int NT, int DQ>
hipError_t launch_ct(const MtArgs &args, int grid, int ct, hipStream_t stream) {
  if (ct == kFP16)
    hipLaunchKernelGGL((gemv_mt_kernel<W, MT, NT, DQ, kFP16>), dim3(grid), dim3(64 * W), 0, stream,
                       args);
  else
    hipLaunchKernelGGL((gemv_mt_kernel<W, MT, NT, DQ, kBF16>), dim3(grid), dim3(64 * W), 0, stream,
                       args);
  return hipGetLastError();
}

template <int W, int MT, int NT>
hipError_t launch_dq(const MtArgs &args, int grid, int dq, int ct, hipStream_t stream) {
  if (dq == kDqCentred) return launch_ct<W, MT, NT, kDqCentred>(args, grid, ct, stream);
  if (dq == kDqSym) return launch_ct<W, MT, NT, kDqSym>(args, grid, ct, stream);
  return launch_ct<W, MT, NT, kDqNone>(args, grid, ct, stream);
}

template <int W, int NT, int CMAX, int D, int DQ, int MT, int BPC>
hipError_t launch_xct(const MtArgs &args, int grid, int ct, hipStream_t stream) {
  if (ct == kFP16)
    hipLaunchKernelGGL((gemv_mtx_kernel<W, NT, CMAX, D, DQ, kFP16, MT, BPC>), dim3(grid),
                       dim3(64 * W), 0, stream, args);
  else
    hipLaunchKernelGGL((gemv_mtx_kernel<W, NT, CMAX, D, DQ, kBF16, MT, BPC>), dim3(grid),
                       dim3(64 * W), 0, stream, args);
  return hipGetLastError();
}

template <int W, int NT, int CMAX, int D, int MT, int BPC>
hipError_t launch_x(const MtArgs &args, int grid, int dq, int ct, hipStream_t stream) {
  if (dq == kDqCentred)
    return launch_xct<W, NT, CMAX, D, kDqCentred, MT, BPC>(args, grid, ct, stream);
  if (dq == kDqSym) return launch_xct<W, NT, CMAX, D, kDqSym, MT, BPC>(args, grid, ct, stream);
  return launch_xct<W, NT, CMAX, D, kDqNone, MT, BPC>(args, grid, ct, stream);
}

// Waves of the register-resident kernel's workgroup by row tiles: 64 activation
// rows take 8 waves with 2 per SIMD (x of two chunks, 128 registers), fewer
// rows 16 waves with 4 per SIMD.
constexpr int xreg_waves(int mt) { return mt == 4 ? 8 : 16; }

// The register-resident kernel for MT row tiles over K ranges of nchs chunks
// (at most xreg_waves(MT) * the x chunks a wave holds), with items in flight
// as registers allow. Staging sized for blocksize 32 takes twice the scale
// registers of blocksize 64 and up, so those take the smaller staging and,
// where that frees the registers, one more item in flight.
template <int BPC>
hipError_t launch_xreg_bpc(const MtArgs &args, int grid, int mt, int cmax, bool long_run, int dq,
                           int ct, hipStream_t stream) {
  if (mt == 4) {
    // a fourth item in flight pays on long item runs (7B layer at M = 64:
    // 89.5 -> 85.6 us) and costs on short ones, whose start-up it lengthens
    // ([11008, 4096] at M = 64: 31.2 -> 33.1 us)
    if (cmax == 2) {
      if constexpr (BPC == 2) {
        if (args.nt == 2) return launch_x<8, 2, 2, 2, 4, BPC>(args, grid, dq, ct, stream);
        if (long_run) return launch_x<8, 1, 2, 4, 4, BPC>(args, grid, dq, ct, stream);
      }
      return launch_x<8, 1, 2, 3, 4, BPC>(args, grid, dq, ct, stream);
    }
    return launch_x<8, 1, 1, 4, 4, BPC>(args, grid, dq, ct, stream);
  }
  if (mt == 2) {
    if (cmax == 2) return launch_x<16, 1, 2, 2, 2, BPC>(args, grid, dq, ct, stream);
    return launch_x<16, 1, 1, 3, 2, BPC>(args, grid, dq, ct, stream);
  }
  // (three items in flight with three chunks measured slower: [4096, 11008]
  // at M = 16, 20.1 -> 22.7 us)
  if (cmax == 3) return launch_x<16, 1, 3, 2, 1, BPC>(args, grid, dq, ct, stream);
  // (a fourth item in flight on the 7B layer at M = 4 / 16 measured 1-6 %
  // slower)
  if (cmax == 2) return launch_x<16, 1, 2, 3, 1, BPC>(args, grid, dq, ct, stream);
  return launch_x<16, 1, 1, 3, 1, BPC>(args, grid, dq, ct, stream);
}

hipError_t launch_xreg(const MtArgs &args, int grid, int mt, int nchs, int dq, int ct,
                       hipStream_t stream) {
  const int cmax = (nchs + xreg_waves(mt) - 1) / xreg_waves(mt);
  const bool long_run = args.total_items >= 12 * grid;  // items per workgroup
  if (args.p[0].log2_bs == 5)
    return launch_xreg_bpc<4>(args, grid, mt, cmax, long_run, dq, ct, stream);
  return launch_xreg_bpc<2>(args, grid, mt, cmax, long_run, dq, ct, stream);
}

// items of 16 nt rows over the launch's problems
int count_items(int count, const GemvDesc *descs, int nt) {
  int items = 0;
  for (int i = 0; i < count; ++i) items += (descs[i].N + 16 * nt - 1) / (16 * nt);
  return items;
}

// The problem fields every kernel reads (the K range is the whole row).
void fill_problem(MtProblem &p, const GemvDesc &d, int M, int K, int dq, uint32_t xe,
                  uint32_t ye) {
  p.x = static_cast<const char *>(d.x);
  p.packed = d.packed;
  p.y = static_cast<char *>(d.y);
  p.bias = static_cast<const char *>(d.bias);
  p.absmax = dq ? d.sc.absmax_scale : d.sc.absmax;
  p.absmax_q = d.sc.absmax_q;
  p.absmax_offset = d.sc.absmax_offset;
  p.N = d.N;
  p.log2_bs = __builtin_ctz((unsigned)d.blocksize);
  p.log2_bs2 = d.sc.log2_bs2;
  p.ldx_bytes = (uint32_t)(d.ldx * xe);
  p.ldy_bytes = (uint32_t)(d.ldy * ye);
  p.x_bytes = (uint32_t)(((int64_t)(M - 1) * d.ldx + K) * xe);
  p.y_bytes = (uint32_t)(((int64_t)(M - 1) * d.ldy + d.N) * ye);
  p.kc0 = 0;
  p.kc1 = (K + kChunk - 1) / kChunk;
  p.jb = 0;
  p.jn = K >> p.log2_bs;
}

void init_args(MtArgs &args, int M, int K, int out_dtype, const CodeTables &tb) {
  args.count = 0;
  args.M = M;
  args.K = K;
  args.out_dtype = out_dtype;
  args.total_items = 0;
  args.nchs = (K + kChunk - 1) / kChunk;
  args.kbs = 0;
  args.nt = 1;
  for (int i = 0; i < kMaxGroup; ++i) args.item_begin[i] = INT_MAX;
  for (int i = 0; i < 16; ++i) args.value[i] = tb.value[i];
}

// Row tiles per item of the register-resident kernel: 64-row launches (8
// waves) at blocksize 64 and up take 32-row items when every workgroup still
// gets at least 6 of them -- half the item ends (barrier and partial-tile
// sums) per weight byte; otherwise, and below 64 rows, 16-row items.
// (the 32-row kernel holds two x chunks per wave: K ranges of 9 to 16 chunks)
int xreg_row_tiles(int count, const GemvDesc *descs, int M, int ranges, int nchs) {
  if (gemv_row_tiles(M) != 4 || descs[0].blocksize < 64 || (nchs + 7) / 8 != 2) return 1;
  return ranges * count_items(count, descs, 2) >= 6 * device_cu_count() ? 2 : 1;
}

// One split launch: products descs[0 .. count) (count * S <= kMaxGroup), each
// as S K ranges writing fp32 partials to its part buffer, then the sums.
hipError_t launch_split(int count, const GemvDesc *descs, float *const *part, int M, int K, int S,
                        int quant_type, int dq, int compute_dtype, int out_dtype,
                        hipStream_t stream) {
  const int mt = gemv_row_tiles(M);
  const int nch = (K + kChunk - 1) / kChunk;
  const int nchs = (nch + S - 1) / S;
  const CodeTables &tb = code_tables(quant_type);
  const uint32_t xe = compute_dtype == kFP32 ? 4u : 2u;
  MtArgs args;
  init_args(args, M, K, kFP32, tb);
  args.nchs = nchs;
  const int nt = xreg_row_tiles(count, descs, M, S, nchs);
  args.nt = nt;
  GemvDesc live[kMaxGroup];
  float *live_part[kMaxGroup];
  int items = 0, nlive = 0;
  for (int i = 0; i < count; ++i) {
    const GemvDesc &d = descs[i];
    if (d.N == 0) continue;
    for (int r = 0; r < S; ++r) {
      const int k = args.count++;
      MtProblem &p = args.p[k];
      fill_problem(p, d, M, K, dq, xe, 4u);
      p.y = reinterpret_cast<char *>(part[i] + (size_t)r * M * d.N);
      p.bias = nullptr;
      p.ldy_bytes = 4u * (uint32_t)d.N;
      p.y_bytes = 4u * (uint32_t)M * (uint32_t)d.N;
      p.kc0 = r * nchs;
      p.kc1 = (r + 1) * nchs < nch ? (r + 1) * nchs : nch;
      const int KB = K >> p.log2_bs;
      p.jb = (p.kc0 * kChunk) >> p.log2_bs;
      const int je = ((p.kc1 * kChunk - 1) >> p.log2_bs) + 1;
      p.jn = (je < KB ? je : KB) - p.jb;
      if (p.jn > args.kbs) args.kbs = p.jn;
      args.item_begin[k] = items;
      p.item_begin = items;
      items += (d.N + 16 * nt - 1) / (16 * nt);
    }
    live[nlive] = d;
    live_part[nlive++] = part[i];
  }
  if (args.count == 0) return hipSuccess;
  args.total_items = items;
  const int cu = device_cu_count();
  const int grid = items < cu ? items : cu;
  hipError_t e = launch_xreg(args, grid, mt, nchs, dq, compute_dtype, stream);
  if (e != hipSuccess) return e;
  int ranges[kMaxGroup];
  for (int i = 0; i < nlive; ++i) ranges[i] = S;
  return launch_gemv_split_sum(nlive, live, live_part, ranges, M, compute_dtype, out_dtype,
                               stream);
}

}  // namespace

hipError_t launch_gemv_split_sum(int count, const GemvDesc *descs, float *const *part,
                                 const int *S, int M, int compute_dtype, int out_dtype,
                                 hipStream_t stream) {
  if (count == 0) return hipSuccess;
  if (count > kMaxGroup) return hipErrorInvalidValue;
  for (int i = 0; i < count; ++i)
    if (S[i] < 1 || S[i] > kMaxSplit) return hipErrorInvalidValue;
  SplitReduceArgs rargs;
  rargs.M = M;
  rargs.out_dtype = out_dtype;
  for (int i = 0; i < kMaxGroup; ++i) rargs.block_begin[i] = INT_MAX;
  int blocks = 0;
  for (int i = 0; i < count; ++i) {
    const GemvDesc &d = descs[i];
    SplitReduceProblem &q = rargs.p[i];
    q.part = part[i];
    q.y = static_cast<char *>(d.y);
    q.bias = static_cast<const char *>(d.bias);
    q.N = d.N;
    q.S = S[i];
    q.ldy_bytes = (uint32_t)(d.ldy * (out_dtype == kFP32 ? 4 : 2));
    q.block_begin = blocks;
    rargs.block_begin[i] = blocks;
    const int64_t quads = (int64_t)M * ((d.N + 3) / 4);
    blocks += (int)((quads + kReduceThreads - 1) / kReduceThreads);
  }
  if (compute_dtype == kFP16)
    hipLaunchKernelGGL((gemv_split_reduce_kernel<kFP16>), dim3(blocks), dim3(kReduceThreads), 0,
                       stream, rargs);
  else
    hipLaunchKernelGGL((gemv_split_reduce_kernel<kBF16>), dim3(blocks), dim3(kReduceThreads), 0,
                       stream, rargs);
  return hipGetLastError();
}

int gemv_max_group() { return kMaxGroup; }

int gemv_row_tiles(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

int gemv_split_ranges(int M, int K) {
  const int nch = (K + kChunk - 1) / kChunk;
  const int mt = gemv_row_tiles(M);
  const int cap = 16 * (mt == 1 ? 3 : (mt == 2 ? 2 : 1));  // chunks of x one CU holds
  const int s = (nch + cap - 1) / cap;
  // up to 8 activation rows the streamed x costs less than the second
  // (summing) launch: on the [4096, 11008] product at M = 4 / 8 streaming took
  // 15.0 / 16.5 us, the split 16.4 / 17.0 us; at M = 16 20.7 vs 18.9 us
  if (s > 1 && M <= 8) return 0;
  return s <= kMaxSplit ? s : 0;
}

// The tiled kernel takes an 8..64-row product whose x the register-resident
// kernel would split into K ranges: two or more ranges at 8..16 rows, three or
// more (or x it could not hold at all) from 17 rows. On [4096, 11008] it
// measured 17.8 / 20.5 / 25.8 us at M = 16 / 32 / 64 against 19.3 / 29-31 /
// 34-35 us; with one or two ranges at 17..64 rows ([11008, 4096]) the two were
// even or the register-resident kernel faster, and a layer launch mixing
// 4096- and 11008-row products slower (more workgroups than one round of CUs).
static bool use_tk(int M, int N, int K) {
  if (M <= 7 || !gemv_tk_enabled() || gemv_tk_ranges(M, N, K) <= 0) return false;
  // 8 rows: where x would take two ranges of the register-resident kernel
  // (which streams x instead at this M); on [4096, 11008] 15.7 against 16.6 us
  if (M == 8) return (K + kChunk - 1) / kChunk > 48;
  const int s = gemv_split_ranges(M, K);
  return M > 16 ? (s == 0 || s >= 3) : s >= 2;
}

size_t gemv_split_bytes(int M, int N, int K) {
  if (use_tk(M, N, K)) return gemv_tk_bytes(M, N, K);
  const int s = gemv_split_ranges(M, K);
  if (s <= 1 || M <= 0 || N <= 0) return 0;
  return ((size_t)s * (size_t)M * (size_t)N * 4u + 255u) & ~(size_t)255u;
}

hipError_t launch_gemv_mt(int count, const GemvDesc *descs, int M, int K, int quant_type, int dq,
                          int compute_dtype, int out_dtype, void *workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  if (count == 0 || M == 0) return hipSuccess;
  if (count > kMaxGroup || M > 64) return hipErrorInvalidValue;
  if (M >= 8) {
    // 8..64 activation rows: the products use_tk picks go to the tiled
    // kernel when the call brings their workspace, the others (a launch of
    // their own, which may use the whole workspace after it) below, so each
    // product takes the kernel it takes alone
    GemvDesc tk[kMaxGroup], rest[kMaxGroup];
    int ntk = 0, nrest = 0;
    size_t tk_need = 0;
    for (int i = 0; i < count; ++i) {
      if (use_tk(M, descs[i].N, K)) {
        tk[ntk++] = descs[i];
        tk_need += gemv_tk_bytes(M, descs[i].N, K);
      } else {
        rest[nrest++] = descs[i];
      }
    }
    if (ntk > 0 && (tk_need == 0 || (workspace != nullptr && workspace_bytes >= tk_need))) {
      const hipError_t e = launch_gemv_tk(ntk, tk, M, K, quant_type, dq, compute_dtype, out_dtype,
                                          workspace, stream);
      if (e != hipSuccess || nrest == 0) return e;
      return launch_gemv_mt(nrest, rest, M, K, quant_type, dq, compute_dtype, out_dtype, workspace,
                            workspace_bytes, stream);
    }
  }
  const int MT = gemv_row_tiles(M);
  const int cu = device_cu_count();
  const int nch = (K + kChunk - 1) / kChunk;
  bool same_bs = true;  // the staged-scale kernel takes one blocksize
  for (int i = 1; i < count; ++i) same_bs = same_bs && descs[i].blocksize == descs[0].blocksize;
  // K ranges on the register-resident kernel (0: too many), and the
  // workspace their partial sums take
  const int S = gemv_split_ranges(M, K);
  size_t need = 0;
  for (int i = 0; i < count; ++i) need += gemv_split_bytes(M, descs[i].N, K);
  bool fits = true;  // 32-bit offsets into each part buffer
  for (int i = 0; i < count; ++i)
    fits = fits && (int64_t)S * M * descs[i].N < ((int64_t)1 << 29);
  if (same_bs && S > 1 && fits && workspace != nullptr && workspace_bytes >= need) {
    if (log_on())
      log_msg("decode M=%d K=%d: gemv_mtx_kernel with %d row tile(s), K split into %d ranges "
              "(%zu workspace bytes), then gemv_split_reduce_kernel; %d product(s)",
              M, K, MT, S, need, count);
    // products in launches of at most kMaxGroup / S, each with its part buffer
    float *part[kMaxGroup];
    char *ws = static_cast<char *>(workspace);
    const int per = kMaxGroup / S;
    for (int i0 = 0; i0 < count; i0 += per) {
      const int c = count - i0 < per ? count - i0 : per;
      for (int i = 0; i < c; ++i) {
        part[i] = reinterpret_cast<float *>(ws);
        ws += gemv_split_bytes(M, descs[i0 + i].N, K);
      }
      const hipError_t e = launch_split(c, descs + i0, part, M, K, S, quant_type, dq,
                                        compute_dtype, out_dtype, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const bool xreg = same_bs && S == 1;
  // streamed kernel: row tiles per item, the most (fewer x fragment loads per
  // weight byte) that still leave every CU a few items; the register budget
  // caps it (4 waves per SIMD at MT = 1 leave 128 registers: NT = 4 would
  // spill). The register-resident kernel takes one row tile per item: its
  // per-item cost is mostly the workgroup's meeting, which grows with the tile.
  int nt = xreg ? xreg_row_tiles(count, descs, M, 1, nch) : 1;
  if (!xreg) {
    const int nt_max = MT == 2 ? 4 : 2;
    for (int c = 2; c <= nt_max; c *= 2)
      if (count_items(count, descs, c) >= 3 * cu) nt = c;
  }
  const CodeTables &tb = code_tables(quant_type);
  MtArgs args;
  init_args(args, M, K, out_dtype, tb);
  const uint32_t xe = compute_dtype == kFP32 ? 4u : 2u;
  const uint32_t ye = out_dtype == kFP32 ? 4u : 2u;
  int items = 0;
  for (int i = 0; i < count; ++i) {
    const GemvDesc &d = descs[i];
    if (d.N == 0) continue;
    const int k = args.count++;
    MtProblem &p = args.p[k];
    fill_problem(p, d, M, K, dq, xe, ye);
    args.item_begin[k] = items;
    p.item_begin = items;
    items += (d.N + 16 * nt - 1) / (16 * nt);
  }
  if (args.count == 0) return hipSuccess;
  args.kbs = args.p[0].jn;
  args.nt = nt;
  args.total_items = items;
  const int grid = items < cu ? items : cu;
  if (log_on())
    log_msg("decode M=%d K=%d: %s, %d row tile(s), %d-row items (%d), grid %d; %d product(s)%s",
            M, K, xreg ? "gemv_mtx_kernel (x in registers)" : "gemv_mt_kernel (x streamed)", MT,
            16 * nt, items, grid, args.count,
            S > 1 && !xreg ? "; a K split needs a workspace of the queried size" : "");
  if (xreg) return launch_xreg(args, grid, MT, nch, dq, compute_dtype, stream);
  if (MT == 1) {
    if (nt == 2) return launch_dq<16, 1, 2>(args, grid, dq, compute_dtype, stream);
    return launch_dq<16, 1, 1>(args, grid, dq, compute_dtype, stream);
  }
  if (MT == 2) {
    if (nt == 4) return launch_dq<8, 2, 4>(args, grid, dq, compute_dtype, stream);
    if (nt == 2) return launch_dq<8, 2, 2>(args, grid, dq, compute_dtype, stream);
    return launch_dq<8, 2, 1>(args, grid, dq, compute_dtype, stream);
  }
  if (nt == 2) return launch_dq<8, 4, 2>(args, grid, dq, compute_dtype, stream);
  return launch_dq<8, 4, 1>(args, grid, dq, compute_dtype, stream);
}

}  // namespace nf4
