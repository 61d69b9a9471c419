// gemm.hip -- prefill product Y[M, N] = X[M, K] . cd(dequant(W))[N, K]^T on
// gfx950 matrix cores, fp32 accumulation; cd is the rounding to the compute
// dtype (bf16 or fp16), the type of X and of the MFMA operands.
//
// [repo page ossradar.top bitsandbytes, release notes 0.50.0: a fused 4-bit
//  dequantize + GEMM replaces dequantize + F.linear; usage page
//  icman.com.cn/news/48546, "Configuration": bf16 compute dtype after 4-bit
//  dequantization.]
//
// Tiling: a workgroup of 8 waves computes a BM x BN = 256 x 224 tile of Y and
// walks K in steps of BK = 64. The waves form a 4 x 2 grid; each owns a
// 64 x 112 sub-tile = 4 x 7 fragments of v_mfma_f32_16x16x32_bf16, whose
// fp32 accumulators stay in registers for the whole K walk.
// Per step two LDS buffers alternate: the MFMAs of step k read one while the
// other is filled for step k+1 --
//  - the X tile goes from memory straight into LDS (buffer loads with the LDS
//    destination), 1 KB per wave instruction, no registers involved;
//  - the weight tile's codes (loaded into registers a step earlier) are
//    dequantized to the same bf16 values the dequantize kernel produces and
//    written to LDS; every thread takes at most one 32-code piece, so the
//    dequantization work is spread over all waves;
// and the codes of step k+2 are loaded. One barrier per step; before it a
// wave waits only for its X loads, not for the code loads issued after them.
// LDS rows are 128 bytes with the 16-byte chunk c of row r stored at chunk
// c ^ ((r / 2) mod 8): the operand reads (16 rows, one chunk each) and the
// row writes then cover every bank once. Staged double-quant scales are held
// block-column-major, so neighbouring rows read neighbouring bytes.
// An optional bias per output column (nf4_linear; compute dtype) is loaded
// before the K walk and added to the fp32 accumulators before the output
// rounding. Rows of X and Y may be strided (ldx, ldy elements).
// Tile order: consecutive workgroups go to different XCDs (8 of them), so
// workgroup i takes M tile i % m_tiles and N tile i / m_tiles: with 8 M tiles
// (M = 2048) each XCD keeps its own X rows hot in its L2 across N tiles.
#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int BM = 256, BN = 224, BK = 64;
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int WM = 4, WN = 2;             // wave grid
constexpr int TM = BM / WM, TN = BN / WN;  // 64 x 112 per wave
constexpr int FM = TM / 16, FN = TN / 16;  // 4 x 7 fragments
constexpr int kStride = BK;                // bf16 per LDS row (128 B, swizzled)
// 16-byte chunk c of tile row r sits at chunk c ^ ((r / 2) mod 8) of its row:
// the 16-byte reads of 16 consecutive rows (one chunk each), and the writes of
// whole rows, then cover every bank once
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kStride + 8 * (chunk ^ ((row >> 1) & 7));
}
constexpr int kWPieces = BN * BK / 32;     // 32-code pieces of the weight tile
constexpr int kWPer = (kWPieces + kThreads - 1) / kThreads;  // weight pieces per thread: 1
constexpr int kBufferFlags = 0x00020000;
constexpr uint32_t kOOB = 0x80000000u;     // an offset past every buffer
// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8):
// all but the newest n memory loads done
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kWaitVm0 = waitcnt_vm(0);
constexpr int kWaitLgkm0 = 15 | (7 << 4) | (3 << 14);  // lgkmcnt(0) only
static_assert(BM * BK * 2 == kWaves * 4 * 1024, "X tile: four 1 KB loads per wave");

struct GemmArgs {
  const uint16_t *x;
  const uint8_t *packed;
  void *y;
  const uint16_t *bias;  // [N] in the compute dtype, or null
  int32_t M, N, K;
  uint32_t ldx, ldy;     // row strides of x and y, elements
  int32_t log2_bs;
  ScaleArgs sc;
  int32_t m_tiles, n_tiles;
  float value[16];
};

// 8 codes of one packed word -> 4 pairs of the compute type in k order,
// through the 16-entry fp32 code table in LDS (byte offsets are 4 * code, cut
// from the word).
template <int CT>
__device__ __forceinline__ uint4 dequant8(uint32_t word, float ap, const char *tb) {
  const uint32_t even4 = (word >> 2) & 0x3c3c3c3cu;  // 4 * high nibble of each byte
  const uint32_t odd4 = (word << 2) & 0x3c3c3c3cu;   // 4 * low nibble of each byte
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float c0 = *reinterpret_cast<const float *>(tb + ((even4 >> (8 * j)) & 0xffu));
    const float c1 = *reinterpret_cast<const float *>(tb + ((odd4 >> (8 * j)) & 0xffu));
    out[j] = pack2<CT>(c0 * ap, c1 * ap);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// SQ: the tile's int8 block scales and group scales are staged in LDS once
// per workgroup (double quant, when they fit), so a step loads only codes.
constexpr int kQStage = 20480;   // int8 block scales of one weight tile
constexpr int kGStage = 512;     // fp32 group scales of one weight tile

template <int DQ, bool SQ, int OUT, int CT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_kernel(GemmArgs args) {
  // memory loads a thread issues per step for the weight tile (codes, plus
  // the block scales when they are not staged in LDS)
  constexpr int kCodeLoads = kWPer * (SQ ? 1 : (DQ == kDqCentred ? 4 : (DQ ? 3 : 2)));
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * kStride];
  // one spare row past the tile: threads without a weight piece (the last
  // wave) write their zeros there, so the step body needs no branch
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][(BN + 1) * kStride];
  __shared__ __attribute__((aligned(16))) float table[16];
  __shared__ __attribute__((aligned(16))) int8_t q_lds[SQ ? kQStage : 1];
  __shared__ __attribute__((aligned(16))) float s2_lds[SQ ? kGStage : 1];
  __shared__ __attribute__((aligned(16))) float mu_lds[SQ && DQ == kDqCentred ? kGStage : 1];
  if (threadIdx.x < 16) table[threadIdx.x] = args.value[threadIdx.x];
  const char *tb = reinterpret_cast<const char *>(table);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int M = args.M, N = args.N, K = args.K;
  const int m_tile = (int)blockIdx.x % args.m_tiles, n_tile = (int)blockIdx.x / args.m_tiles;
  const int m0 = m_tile * BM, n0 = n_tile * BN;
  const int nk = (K + BK - 1) / BK;
  const uint32_t row_bytes = (uint32_t)K >> 1;

  const int x_rows = M - m0 < BM ? M - m0 : BM;
  const uint32_t ldx = args.ldx;
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(args.x + (int64_t)m0 * ldx), (short)0,
      (int)(2u * ((uint32_t)(x_rows - 1) * ldx + (uint32_t)K)), kBufferFlags);
  // weight tile: piece p = tid + kThreads * u (< kWPieces) is row p / 2,
  // 32-code half p % 2
  const int w_rows = N - n0 < BN ? N - n0 : BN;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(args.packed + (int64_t)n0 * row_bytes), (short)0,
      (int)((uint32_t)w_rows * row_bytes), kBufferFlags);
  // block scales of the tile's rows: byte/float offsets relative to the tile's
  // first block; the group scale relative to its group (64-bit safe)
  const uint32_t row_blocks = (uint32_t)K >> args.log2_bs;
  const uint64_t blk0 = (uint64_t)n0 * row_blocks;
  const uint32_t tile_blocks = (uint32_t)w_rows * row_blocks;
  const int log2_bs2 = args.sc.log2_bs2;
  const uint64_t gbase = blk0 >> log2_bs2;
  const uint32_t blk_in = (uint32_t)(blk0 & (((uint64_t)1 << log2_bs2) - 1));
  // the groups the tile's blocks fall in
  const uint32_t groups = (blk_in + tile_blocks + (1u << log2_bs2) - 1) >> log2_bs2;
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      DQ ? (void *)(args.sc.absmax_q + blk0) : (void *)(args.sc.absmax + blk0), (short)0,
      (int)(DQ ? tile_blocks : 4u * tile_blocks), kBufferFlags);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      DQ ? (void *)(args.sc.absmax_scale + gbase) : (void *)args.sc.absmax, (short)0,
      (int)(DQ ? 4u * groups : 0u), kBufferFlags);
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      DQ == kDqCentred ? (void *)(args.sc.absmax_offset + gbase) : (void *)args.sc.absmax,
      (short)0, (int)(DQ == kDqCentred ? 4u * groups : 0u), kBufferFlags);

  uint4 wr[kWPer];
  float w_scale[kWPer];
  uint32_t w_blk[kWPer];
  auto load_step = [&](int ks) {
    const int k0 = ks * BK;
    {
#pragma unroll
      for (int u = 0; u < kWPer; ++u) {
        const int p = tid + kThreads * u;
        const int row = p >> 1, kc = k0 + 32 * (p & 1);
        const bool ok = p < kWPieces && row < w_rows && kc < K;
        const uint32_t off = ok ? (uint32_t)row * row_bytes + ((uint32_t)kc >> 1) : kOOB;
        wr[u] =
            __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)off, 0, 0));
        // the 32 codes lie in one block; out of range: scale 0
        const uint32_t blk = (uint32_t)row * row_blocks + ((uint32_t)kc >> args.log2_bs);
        if (SQ) {
          w_blk[u] = ok ? blk : 0xffffffffu;  // the scale is read from LDS at dequant
        } else if (DQ) {
          const int q =
              (int8_t)__builtin_amdgcn_raw_buffer_load_b8(qrs, (int)(ok ? blk : kOOB), 0, 0);
          const uint32_t goff = ok ? ((blk_in + blk) >> log2_bs2) << 2 : kOOB;
          const float s2 = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(srs, (int)goff, 0, 0));
          const float mu = DQ == kDqCentred
                               ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                               mrs, (int)goff, 0, 0))
                               : 0.0f;
          w_scale[u] = scale_from<DQ>(q, s2, mu);
        } else {
          w_scale[u] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(qrs, (int)(ok ? blk << 2 : kOOB), 0, 0));
        }
      }
    }
  };
  // X tile straight from memory into LDS: wave w fills rows 32 w .. 32 w + 31,
  // 8 rows (1 KB) per instruction; lane 8 r' + q of an instruction lands at
  // position q of its row r, so it fetches the chunk that the swizzle puts
  // there. Rows past M and columns past K read zeros.
  auto x_direct = [&](int ks, int buf) {
    const int k0 = ks * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (4 * wave + i) * 8 + (lane >> 3), q = lane & 7;
      const int c = q ^ ((r >> 1) & 7);
      const int kc = k0 + 8 * c;
      const uint32_t off = kc < K ? 2u * ((uint32_t)r * ldx + (uint32_t)kc) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrs, (__attribute__((address_space(3))) void *)&xs[buf][(4 * wave + i) * 512], 16,
          (int)off, 0, 0, 0);
    }
  };
  auto store_step = [&](int buf) {
    {
#pragma unroll
      for (int u = 0; u < kWPer; ++u) {
        const int p = tid + kThreads * u;
        // pieces past the tile go to the spare row
        const int wrow = p < kWPieces ? p >> 1 : BN, wc = 4 * (p & 1);
        uint16_t *wbase = ws[buf];
        float ap = w_scale[u];
        if (SQ) {
          // q_lds holds the tile's int8 scales block-column-major (row
          // fastest), so the rows of one wave read neighbouring bytes
          const bool ok = w_blk[u] != 0xffffffffu;
          const uint32_t b = ok ? w_blk[u] : 0u;
          const uint32_t row = (uint32_t)(p >> 1), kb = b - row * row_blocks;
          const uint32_t gi = (blk_in + b) >> log2_bs2;
          ap = ok ? scale_from<DQ>(q_lds[kb * BN + row], s2_lds[gi],
                                   DQ == kDqCentred ? mu_lds[gi] : 0.0f)
                  : 0.0f;
        }
        *reinterpret_cast<uint4 *>(wbase + swz(wrow, wc + 0)) = dequant8<CT>(wr[u].x, ap, tb);
        *reinterpret_cast<uint4 *>(wbase + swz(wrow, wc + 1)) = dequant8<CT>(wr[u].y, ap, tb);
        *reinterpret_cast<uint4 *>(wbase + swz(wrow, wc + 2)) = dequant8<CT>(wr[u].z, ap, tb);
        *reinterpret_cast<uint4 *>(wbase + swz(wrow, wc + 3)) = dequant8<CT>(wr[u].w, ap, tb);
      }
    }
  };

  // bias of this lane's output columns n0 + wn * TN + 16 j + lane % 16 (a
  // column past N reads 0 through the buffer's range check)
  const bool has_bias = args.bias != nullptr;
  float bias_n[FN];
  {
    const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)args.bias, (short)0, has_bias ? (int)(2u * (uint32_t)N) : 0, kBufferFlags);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * TN + 16 * j + (lane & 15);
      bias_n[j] = widen16<CT>(
          __builtin_amdgcn_raw_buffer_load_b16(brs, (int)(2u * (uint32_t)n), 0, 0));
    }
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (SQ) {
    // the tile's block scales (tile_blocks bytes, contiguous) and the group
    // scales they use (groups floats, contiguous)
    for (uint32_t i = tid; i < tile_blocks; i += kThreads) {
      const uint32_t row = i / row_blocks, kb = i - row * row_blocks;
      q_lds[kb * BN + row] = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(qrs, (int)i, 0, 0);
    }
    for (uint32_t i = tid; i < groups; i += kThreads) {
      s2_lds[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, (int)(4 * i), 0, 0));
      if (DQ == kDqCentred)
        mu_lds[i] =
            __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(mrs, (int)(4 * i), 0, 0));
    }
  }
  __syncthreads();  // code table, staged scales
  x_direct(0, 0);
  load_step(0);
  store_step(0);
  load_step(1 < nk ? 1 : nk - 1);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();

  // operand rows of this lane: A row wm*64 + 16 fi + lane%16, B row
  // wn*112 + 16 fj + lane%16; k = 32 h + 8 (lane / 16)
  const int lr = lane & 15, lc = lane >> 4;
  // Step ks: the MFMAs of step ks read buffer ks % 2. Meanwhile the X tile of
  // step ks + 1 streams into the other buffer, the weight codes of step
  // ks + 1 (in registers since the previous step) are dequantized into it,
  // and the codes of step ks + 2 are loaded. Before the step's barrier the
  // wave waits for its X loads (older than the code loads), not for the code
  // loads issued after them.
  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    x_direct(ks + 1 < nk ? ks + 1 : nk - 1, cur ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    store_step(cur ^ 1);
    load_step(ks + 2 < nk ? ks + 2 : nk - 1);
    // both halves' operands first, so the reads of the second half overlap
    // the first half's matrix-core work
    uint4 a[2][FM], b[2][FN];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[h][i] = *reinterpret_cast<const uint4 *>(&xs[cur][swz(wm * TM + 16 * i + lr, 4 * h + lc)]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[h][j] = *reinterpret_cast<const uint4 *>(&ws[cur][swz(wn * TN + 16 * j + lr, 4 * h + lc)]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32<CT>(a[h][i], b[h][j], acc[i][j]);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kCodeLoads));
    __syncthreads();
  }

  // D layout of the 16x16 MFMA: lane l holds column l % 16 and rows
  // 4 (l / 16) + r. Stores go through a buffer resource: rows past M and
  // columns past N get an out-of-range offset and are dropped. The bias of
  // the lane's columns (loaded before the K walk) is added in fp32.
  constexpr uint32_t kOut = OUT == kFP32 ? 4u : 2u;
  const uint32_t ldy = args.ldy;
  const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((char *)args.y + (int64_t)m0 * ldy * kOut), (short)0,
      (int)(((uint32_t)(x_rows - 1) * ldy + (uint32_t)N) * kOut), kBufferFlags);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * TN + 16 * j + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = wm * TM + 16 * i + 4 * (lane >> 4) + r;  // row within the tile
        const uint32_t off = (n < N && m < x_rows) ? ((uint32_t)m * ldy + (uint32_t)n) * kOut : kOOB;
        // (a scalar copy first: a bit cast of a vector element directly
        // has been compiled as a cast of element 0)
        const float v = has_bias ? acc[i][j][r] + bias_n[j] : acc[i][j][r];
        if (OUT != kFP32)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)out_bits<OUT>(v), yrs, (int)off, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), yrs, (int)off, 0,
                                                0);
      }
    }
}

template <int DQ, bool SQ, int CT>
hipError_t launch_cfg(const GemmArgs &args, int grid, int out_dtype, hipStream_t stream) {
  if (out_dtype == kFP32)
    hipLaunchKernelGGL((gemm_kernel<DQ, SQ, kFP32, CT>), dim3(grid), dim3(kThreads), 0, stream, args);
  else if (out_dtype == kFP16)
    hipLaunchKernelGGL((gemm_kernel<DQ, SQ, kFP16, CT>), dim3(grid), dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((gemm_kernel<DQ, SQ, kBF16, CT>), dim3(grid), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

template <int CT>
hipError_t launch_ct(const GemmArgs &args, int grid, int out_dtype, int blocksize,
                     hipStream_t stream) {
  const ScaleArgs &sc = args.sc;
  if (!sc.double_quant) return launch_cfg<kDqNone, false, CT>(args, grid, out_dtype, stream);
  // a tile's scales fit in LDS: at most kQStage blocks, and the groups they
  // touch (one more than they fill, at most) within kGStage
  const int64_t tile_blocks = (int64_t)BN * (args.K / blocksize);
  const int64_t groups = tile_blocks / (1 << sc.log2_bs2) + 2;
  const bool sq = tile_blocks <= kQStage && groups <= kGStage;
  if (sc.double_quant == kDqCentred)
    return sq ? launch_cfg<kDqCentred, true, CT>(args, grid, out_dtype, stream)
              : launch_cfg<kDqCentred, false, CT>(args, grid, out_dtype, stream);
  return sq ? launch_cfg<kDqSym, true, CT>(args, grid, out_dtype, stream)
            : launch_cfg<kDqSym, false, CT>(args, grid, out_dtype, stream);
}

// ---------------------------------------------------------------------------
// The product on weights already in the compute dtype: w16 [N, K], rows ldw
// elements apart (the dequantize kernel's output). Same tiles, wave grid and
// MFMA order as gemm_kernel, so the result is bitwise gemm_kernel's on the
// weight w16 was dequantized from; what differs is the pipeline. Both tiles
// stream into LDS with no register round trip, in 32-deep steps through four
// LDS stages, and a wave reads the next step's operands while its MFMAs run
// on the current ones:
//  - step ks issues the loads of step ks + 3 (into the stage step ks - 1
//    used), reads step ks + 1's operands from LDS and runs step ks's MFMAs on
//    operands it read during step ks - 1; one barrier per step, before which
//    a wave waits for its loads of step ks + 2;
//  - a stage is 256 rows of X and 256 rows of weights (the last 32 zero) of
//    64 bytes; 16-byte chunk c of row r sits at chunk c ^ ((r / 2) mod 4), so
//    each 8 lanes of an operand read (8 rows x 16 bytes) cover all 32 banks
//    (a timing probe of the read patterns: this one as fast as linear reads,
//    c ^ ((r / 4) mod 4) or no swizzle 1.75 times slower);
//  - waves 0-3 load the X tile, waves 4-7 the weight tile, four 1 KB loads
//    each per step.
constexpr int BK2 = 32;
constexpr int kStages = 4;

__device__ __forceinline__ int swz2(int row, int chunk) {
  return row * BK2 + 8 * (chunk ^ ((row >> 1) & 3));
}

struct GemmW16Args {
  const uint16_t *x;
  const uint16_t *w16;
  void *y;
  const uint16_t *bias;  // [N] in the compute dtype, or null
  int32_t M, N, K;
  uint32_t ldx, ldw, ldy;
  int32_t m_tiles, n_tiles;
  int32_t panels_by_xcd;  // n_tiles % 8 == 0: each XCD takes whole weight panels
};

template <int OUT, int CT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_w16_kernel(GemmW16Args args) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kStages][BM * BK2];
  __shared__ __attribute__((aligned(16))) uint16_t ws[kStages][BM * BK2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int M = args.M, N = args.N, K = args.K;
  // Consecutive workgroups go to the 8 XCDs in turn. With whole panels per
  // XCD, XCD x takes weight panels x, x + 8, ... with every M tile of each, so
  // a panel streams from memory into one XCD's L2 and its M tiles share it;
  // otherwise M tiles vary fastest.
  int m_tile, n_tile;
  if (args.panels_by_xcd) {
    const int xcd = (int)blockIdx.x & 7, jj = (int)blockIdx.x >> 3;
    m_tile = jj % args.m_tiles;
    n_tile = (jj / args.m_tiles) * 8 + xcd;
  } else {
    m_tile = (int)blockIdx.x % args.m_tiles;
    n_tile = (int)blockIdx.x / args.m_tiles;
  }
  const int m0 = m_tile * BM, n0 = n_tile * BN;
  const int nk = (K + BK2 - 1) / BK2;
  const int x_rows = M - m0 < BM ? M - m0 : BM;
  const int w_rows = N - n0 < BN ? N - n0 : BN;
  const uint32_t ldx = args.ldx, ldw = args.ldw;
  // waves 0-3: X rows, waves 4-7: weight rows; rows past the matrix read zeros
  const bool x_side = wave < 4;
  const __amdgpu_buffer_rsrc_t rs = x_side
      ? __builtin_amdgcn_make_buffer_rsrc(
            (void *)(args.x + (int64_t)m0 * ldx), (short)0,
            (int)(2u * ((uint32_t)(x_rows - 1) * ldx + (uint32_t)K)), kBufferFlags)
      : __builtin_amdgcn_make_buffer_rsrc(
            (void *)(args.w16 + (int64_t)n0 * ldw), (short)0,
            (int)(2u * ((uint32_t)(w_rows - 1) * ldw + (uint32_t)K)), kBufferFlags);
  const uint32_t ld = x_side ? ldx : ldw;
  const int row_cap = x_side ? BM : BN;
  // this wave's four loads of step ks into stage st: load i covers tile rows
  // 16 t .. 16 t + 15 with t = 4 (wave mod 4) + i, lane 4 r' + p landing at
  // chunk p of row 16 t + r' (so it fetches the chunk the swizzle puts
  // there); steps past K read zeros (offsets past the buffer)
  auto fill = [&](int ks, int st) {
    const int k0 = ks * BK2;
    uint16_t *base = x_side ? xs[st] : ws[st];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * (wave & 3) + i;
      const int r = 16 * t + (lane >> 2), p = lane & 3;
      const int kc = k0 + 8 * (p ^ ((r >> 1) & 3));
      const uint32_t off = (ks < nk && kc < K && r < row_cap) ? 2u * ((uint32_t)r * ld + (uint32_t)kc)
                                                             : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void *)(base + t * 512), 16, (int)off, 0, 0, 0);
    }
  };

  const bool has_bias = args.bias != nullptr;
  float bias_n[FN];
  {
    const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)args.bias, (short)0, has_bias ? (int)(2u * (uint32_t)N) : 0, kBufferFlags);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * TN + 16 * j + (lane & 15);
      bias_n[j] = widen16<CT>(
          __builtin_amdgcn_raw_buffer_load_b16(brs, (int)(2u * (uint32_t)n), 0, 0));
    }
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // operand rows of this lane: A row wm*64 + 16 i + lane%16, B row
  // wn*112 + 16 j + lane%16, k chunk lane / 16
  const int lr = lane & 15, lc = lane >> 4;
  auto read_ops = [&](int st, uint4 (&a)[FM], uint4 (&b)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      a[i] = *reinterpret_cast<const uint4 *>(&xs[st][swz2(wm * TM + 16 * i + lr, lc)]);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      b[j] = *reinterpret_cast<const uint4 *>(&ws[st][swz2(wn * TN + 16 * j + lr, lc)]);
  };
  auto mfmas = [&](const uint4 (&a)[FM], const uint4 (&b)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32<CT>(a[i], b[j], acc[i][j]);
  };
  // one step: loads of step ks + 3, operands of step ks + 1 into (an, bn),
  // MFMAs of step ks from (ac, bc); then the wait for this wave's loads of
  // step ks + 2 (all but the four just issued) and the barrier
  auto step = [&](int ks, const uint4 (&ac)[FM], const uint4 (&bc)[FN], uint4 (&an)[FM],
                  uint4 (&bn)[FN]) {
    fill(ks + kStages - 1, (ks + kStages - 1) % kStages);
    // (at the last step this reads a stage that is not used again)
    read_ops((ks + 1) % kStages, an, bn);
    mfmas(ac, bc);
    // issue order: the loads and operand reads each behind one MFMA, so the
    // matrix core starts right after the barrier and the reads complete under
    // the MFMAs; all MFMAs ahead of the wait (the scheduler would otherwise
    // sink them past the barrier and make them wait for these reads)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one memory load
    }
#pragma unroll
    for (int i = 0; i < FM + FN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - 4 - FM - FN, 0);
    __builtin_amdgcn_sched_barrier(0);
    // this step's operand reads and the loads of step ks + 2 done, then a bare
    // barrier: a workgroup fence would make the compiler wait for every load
    // in flight, the ones just issued included
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * (kStages - 3)) & ~(15 << 8));
    __builtin_amdgcn_s_barrier();
  };

#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) fill(s, s);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  uint4 a0[FM], b0[FN], a1[FM], b1[FN];
  read_ops(0, a0, b0);
  // (waited here, so the loop's first MFMAs do not count these reads as
  // possibly in flight on every later trip)
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  int ks = 0;
  for (; ks + 1 < nk; ks += 2) {
    step(ks, a0, b0, a1, b1);
    step(ks + 1, a1, b1, a0, b0);
  }
  if (ks < nk) mfmas(a0, b0);

  constexpr uint32_t kOut = OUT == kFP32 ? 4u : 2u;
  const uint32_t ldy = args.ldy;
  const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((char *)args.y + (int64_t)m0 * ldy * kOut), (short)0,
      (int)(((uint32_t)(x_rows - 1) * ldy + (uint32_t)N) * kOut), kBufferFlags);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * TN + 16 * j + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = wm * TM + 16 * i + 4 * (lane >> 4) + r;
        const uint32_t off = (n < N && m < x_rows) ? ((uint32_t)m * ldy + (uint32_t)n) * kOut : kOOB;
        const float v = has_bias ? acc[i][j][r] + bias_n[j] : acc[i][j][r];
        if (OUT != kFP32)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)out_bits<OUT>(v), yrs, (int)off, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), yrs, (int)off, 0,
                                                0);
      }
    }
}

template <int CT>
hipError_t launch_w16_ct(const GemmW16Args &args, int grid, int out_dtype, hipStream_t stream) {
  if (out_dtype == kFP32)
    hipLaunchKernelGGL((gemm_w16_kernel<kFP32, CT>), dim3(grid), dim3(kThreads), 0, stream, args);
  else if (out_dtype == kFP16)
    hipLaunchKernelGGL((gemm_w16_kernel<kFP16, CT>), dim3(grid), dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((gemm_w16_kernel<kBF16, CT>), dim3(grid), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const void *x, int64_t ldx, int M, const uint8_t *packed, int N, int K,
                       int blocksize, int quant_type, const ScaleArgs &sc, int compute_dtype,
                       int out_dtype, void *y, int64_t ldy, const void *bias, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const CodeTables &t = code_tables(quant_type);
  GemmArgs args;
  args.x = static_cast<const uint16_t *>(x);
  args.packed = packed;
  args.y = y;
  args.bias = static_cast<const uint16_t *>(bias);
  args.M = M;
  args.N = N;
  args.K = K;
  args.ldx = (uint32_t)ldx;
  args.ldy = (uint32_t)ldy;
  args.log2_bs = __builtin_ctz((unsigned)blocksize);
  args.sc = sc;
  args.m_tiles = (M + BM - 1) / BM;
  args.n_tiles = (N + BN - 1) / BN;
  for (int i = 0; i < 16; ++i) args.value[i] = t.value[i];
  const int64_t grid = (int64_t)args.m_tiles * args.n_tiles;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (compute_dtype == kFP16) return launch_ct<kFP16>(args, (int)grid, out_dtype, blocksize, stream);
  return launch_ct<kBF16>(args, (int)grid, out_dtype, blocksize, stream);
}

hipError_t launch_gemm_w16(const void *x, int64_t ldx, int M, const void *w16, int64_t ldw, int N,
                           int K, int compute_dtype, int out_dtype, void *y, int64_t ldy,
                           const void *bias, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmW16Args args;
  args.x = static_cast<const uint16_t *>(x);
  args.w16 = static_cast<const uint16_t *>(w16);
  args.y = y;
  args.bias = static_cast<const uint16_t *>(bias);
  args.M = M;
  args.N = N;
  args.K = K;
  args.ldx = (uint32_t)ldx;
  args.ldw = (uint32_t)ldw;
  args.ldy = (uint32_t)ldy;
  args.m_tiles = (M + BM - 1) / BM;
  args.n_tiles = (N + BN - 1) / BN;
  args.panels_by_xcd = args.n_tiles % 8 == 0;
  const int64_t grid = (int64_t)args.m_tiles * args.n_tiles;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (compute_dtype == kFP16) return launch_w16_ct<kFP16>(args, (int)grid, out_dtype, stream);
  return launch_w16_ct<kBF16>(args, (int)grid, out_dtype, stream);
}

}  // namespace nf4
