// gemm.hip -- prefill product Y[M, N] = X[M, K] . bf16(dequant(W))[N, K]^T on
// gfx950 bf16 matrix cores, fp32 accumulation.
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
// Per step the X tile (bf16) and the weight tile -- read as packed codes and
// dequantized on the fly to the same bf16 values the dequantize kernel
// produces -- are written to one of two LDS buffers while the matrix cores
// work on the other: the global loads of step k+1 are issued before the
// MFMAs of step k, the dequantization and LDS writes follow them, and one
// barrier per step separates the two buffers. LDS rows are padded by 16
// bytes, so the 16-byte operand reads of 16 consecutive lanes (16 rows) cover
// all 64 banks once.
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
constexpr int kStride = BK + 8;            // bf16 per LDS row (144 B)
constexpr int kXPieces = BM * BK / 8;      // 16-byte pieces of the X tile
constexpr int kWPieces = BN * BK / 32;     // 32-code pieces of the weight tile
// Waves 0-3 (one per SIMD) stage and dequantize the weight tile, waves 4-7
// stage the X tile; all eight run MFMAs, so on every SIMD the matrix-core
// work of one wave overlaps the dequantization of the other.
constexpr int kHalf = kThreads / 2;
constexpr int kXPer = kXPieces / kHalf;                  // 8
constexpr int kWPer = (kWPieces + kHalf - 1) / kHalf;    // 2
constexpr int kBufferFlags = 0x00020000;
constexpr uint32_t kOOB = 0x80000000u;     // an offset past every buffer
static_assert(kXPieces % kHalf == 0, "X tile pieces per thread");

struct GemmArgs {
  const uint16_t *x;
  const uint8_t *packed;
  void *y;
  int32_t M, N, K;
  int32_t log2_bs;
  ScaleArgs sc;
  int32_t m_tiles, n_tiles;
  float value[16];
};

// 8 codes of one packed word -> 4 bf16 pairs in k order, through the 16-entry
// fp32 code table in LDS (byte offsets are 4 * code, cut from the word).
__device__ __forceinline__ uint4 dequant8(uint32_t word, float ap, const char *tb) {
  const uint32_t even4 = (word >> 2) & 0x3c3c3c3cu;  // 4 * high nibble of each byte
  const uint32_t odd4 = (word << 2) & 0x3c3c3c3cu;   // 4 * low nibble of each byte
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float c0 = *reinterpret_cast<const float *>(tb + ((even4 >> (8 * j)) & 0xffu));
    const float c1 = *reinterpret_cast<const float *>(tb + ((odd4 >> (8 * j)) & 0xffu));
    out[j] = pack_bf16x2(c0 * ap, c1 * ap);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// SQ: the tile's int8 block scales and group scales are staged in LDS once
// per workgroup (double quant, when they fit), so a step loads only codes.
constexpr int kQStage = 20480;   // int8 block scales of one weight tile
constexpr int kGStage = 512;     // fp32 group scales of one weight tile

template <bool DQ, bool SQ, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * kStride];
  // one spare row past the tile: threads without a weight piece (the last
  // wave) write their zeros there, so the step body needs no branch
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][(BN + 1) * kStride];
  __shared__ __attribute__((aligned(16))) float table[16];
  __shared__ __attribute__((aligned(16))) int8_t q_lds[SQ ? kQStage : 1];
  __shared__ __attribute__((aligned(16))) float s2_lds[SQ ? kGStage : 1];
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

  // X tile (waves 4-7): piece p = xt + kHalf * i is row p / 8, k chunk p % 8.
  const bool x_role = wave >= 4;
  const int xt = tid - kHalf;
  const int x_rows = M - m0 < BM ? M - m0 : BM;
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(args.x + (int64_t)m0 * K), (short)0, (int)(2u * (uint32_t)x_rows * (uint32_t)K),
      kBufferFlags);
  // weight tile (waves 0-3): piece p = tid + kHalf * u (< kWPieces) is row
  // p / 2, 32-code half p % 2
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

  uint4 xr[kXPer];
  uint4 wr[kWPer];
  float w_scale[kWPer];
  uint32_t w_blk[kWPer];
  auto load_step = [&](int ks) {
    const int k0 = ks * BK;
    if (x_role) {
#pragma unroll
      for (int i = 0; i < kXPer; ++i) {
        const int p = xt + kHalf * i;
        const int row = p >> 3, kc = k0 + 8 * (p & 7);
        const uint32_t off = kc < K ? 2u * ((uint32_t)row * (uint32_t)K + (uint32_t)kc) : kOOB;
        xr[i] =
            __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)off, 0, 0));
      }
    } else {
#pragma unroll
      for (int u = 0; u < kWPer; ++u) {
        const int p = tid + kHalf * u;
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
          const float s2 = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(
                         srs, (int)(ok ? ((blk_in + blk) >> log2_bs2) << 2 : kOOB), 0, 0));
          w_scale[u] = (float)q * s2;
        } else {
          w_scale[u] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(qrs, (int)(ok ? blk << 2 : kOOB), 0, 0));
        }
      }
    }
  };
  auto store_step = [&](int buf) {
    if (x_role) {
      uint16_t *xb = xs[buf];
#pragma unroll
      for (int i = 0; i < kXPer; ++i) {
        const int p = xt + kHalf * i;
        *reinterpret_cast<uint4 *>(&xb[(p >> 3) * kStride + 8 * (p & 7)]) = xr[i];
      }
    } else {
#pragma unroll
      for (int u = 0; u < kWPer; ++u) {
        const int p = tid + kHalf * u;
        // pieces past the tile go to the spare row
        uint16_t *wb = &ws[buf][(p < kWPieces ? p >> 1 : BN) * kStride + 32 * (p & 1)];
        float ap = w_scale[u];
        if (SQ) {
          const bool ok = w_blk[u] != 0xffffffffu;
          const uint32_t b = ok ? w_blk[u] : 0u;
          ap = ok ? (float)q_lds[b] * s2_lds[(blk_in + b) >> log2_bs2] : 0.0f;
        }
        *reinterpret_cast<uint4 *>(wb + 0) = dequant8(wr[u].x, ap, tb);
        *reinterpret_cast<uint4 *>(wb + 8) = dequant8(wr[u].y, ap, tb);
        *reinterpret_cast<uint4 *>(wb + 16) = dequant8(wr[u].z, ap, tb);
        *reinterpret_cast<uint4 *>(wb + 24) = dequant8(wr[u].w, ap, tb);
      }
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (SQ) {
    // the tile's block scales (tile_blocks bytes, contiguous) and the group
    // scales they use (groups floats, contiguous)
    for (uint32_t i = tid; i < tile_blocks; i += kThreads)
      q_lds[i] = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(qrs, (int)i, 0, 0);
    for (uint32_t i = tid; i < groups; i += kThreads)
      s2_lds[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, (int)(4 * i), 0, 0));
  }
  __syncthreads();  // code table, staged scales
  load_step(0);
  store_step(0);
  load_step(1 < nk ? 1 : nk - 1);
  __syncthreads();

  // operand rows of this lane: A row wm*64 + 16 fi + lane%16, B row
  // wn*112 + 16 fj + lane%16; k = 32 h + 8 (lane / 16)
  const int lr = lane & 15, lk = 8 * (lane >> 4);
  // Step ks: the MFMAs of step ks read buffer ks % 2 while step ks + 1 --
  // loaded into registers during the previous step -- is dequantized into
  // the other buffer, then the loads of step ks + 2 are issued. One basic
  // block per step (no branches: past the last step the loads repeat it and
  // the writes go to the buffer no one reads any more), so the scheduler can
  // interleave the dequantization with the matrix-core work.
  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    store_step(cur ^ 1);
    load_step(ks + 2 < nk ? ks + 2 : nk - 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4 *>(
                        &xs[cur][(wm * TM + 16 * i + lr) * kStride + 32 * h + lk]));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[j] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4 *>(
                        &ws[cur][(wn * TN + 16 * j + lr) * kStride + 32 * h + lk]));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // D layout of the 16x16 MFMA: lane l holds column l % 16 and rows
  // 4 (l / 16) + r. Stores go through a buffer resource: rows past M and
  // columns past N get an out-of-range offset and are dropped.
  constexpr uint32_t kOut = OUT_BF16 ? 2u : 4u;
  const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((char *)args.y + (int64_t)m0 * N * kOut), (short)0,
      (int)((uint32_t)x_rows * (uint32_t)N * kOut), kBufferFlags);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * TN + 16 * j + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = wm * TM + 16 * i + 4 * (lane >> 4) + r;  // row within the tile
        const uint32_t off = n < N ? ((uint32_t)m * (uint32_t)N + (uint32_t)n) * kOut : kOOB;
        // (a scalar copy first: a bit cast of a vector element directly
        // has been compiled as a cast of element 0)
        const float v = acc[i][j][r];
        if (OUT_BF16)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu), yrs,
                                                (int)off, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), yrs, (int)off, 0,
                                                0);
      }
    }
}

template <bool DQ, bool SQ>
hipError_t launch_cfg(const GemmArgs &args, int grid, bool out_bf16, hipStream_t stream) {
  if (out_bf16)
    hipLaunchKernelGGL((gemm_kernel<DQ, SQ, true>), dim3(grid), dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((gemm_kernel<DQ, SQ, false>), dim3(grid), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint16_t *x, int M, const uint8_t *packed, int N, int K,
                       int blocksize, int quant_type, const ScaleArgs &sc, bool out_bf16,
                       void *y, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const CodeTables &t = code_tables(quant_type);
  GemmArgs args;
  args.x = x;
  args.packed = packed;
  args.y = y;
  args.M = M;
  args.N = N;
  args.K = K;
  args.log2_bs = __builtin_ctz((unsigned)blocksize);
  args.sc = sc;
  args.m_tiles = (M + BM - 1) / BM;
  args.n_tiles = (N + BN - 1) / BN;
  for (int i = 0; i < 16; ++i) args.value[i] = t.value[i];
  const int64_t grid = (int64_t)args.m_tiles * args.n_tiles;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (sc.absmax_q == nullptr) return launch_cfg<false, false>(args, (int)grid, out_bf16, stream);
  // a tile's scales fit in LDS: at most kQStage blocks, and the groups they
  // touch (one more than they fill, at most) within kGStage
  const int64_t tile_blocks = (int64_t)BN * (K / blocksize);
  const int64_t groups = tile_blocks / (1 << sc.log2_bs2) + 2;
  if (tile_blocks <= kQStage && groups <= kGStage)
    return launch_cfg<true, true>(args, (int)grid, out_bf16, stream);
  return launch_cfg<true, false>(args, (int)grid, out_bf16, stream);
}

}  // namespace nf4
