// gemv_tk.hip -- decode products y_i[M, N_i] = x_i[M, K] . cd(dequant(W_i))^T
// for 8 <= M <= 64 on gfx950 matrix cores, with x staged through LDS and the
// K dimension split over workgroups; cd is the rounding to the compute dtype
// (bf16 or fp16).
//
// [repo page ossradar.top bitsandbytes, release notes 0.50.0: 4-bit inference
//  at batch 2..64 uses a fused 4-bit dequantize + GEMM chosen at run time from
//  the shape and the number of compute units, with nested (double)
//  quantization and the bias fused in; usage page icman.com.cn/news/48546,
//  "Configuration": weights are dequantized to the compute dtype.]
//
// Why a second decode kernel. Once x of a long row no longer fits the
// registers of a CU, a kernel that splits K over the waves of a workgroup
// pays, for every 16-row item, a meeting of all its waves whose LDS traffic
// grows with M (at M = 64 four times the item's code bytes). Here no wave
// shares an output with another wave of its group:
//  - a workgroup (8 waves) owns a block of weight rows over one K range of
//    nchs 128-code chunks; the waves form two groups that take the even and
//    the odd chunks of the range, and each wave of a group owns a quarter of
//    the block's rows over all of its group's chunks, so partial sums meet
//    once per workgroup, at its end. Up to 16 activation rows a block is 64
//    rows (one 16-row MFMA tile per wave; under 100 registers and 80 KB of
//    LDS, so two workgroups share a CU and overlap their step chains), above
//    that 128 rows (two tiles per wave, one workgroup per CU);
//  - x of a pair of chunks (both groups' steps) is loaded by all 512 threads
//    with coalesced 16-byte loads, three steps ahead, and written to one of
//    two LDS stages; the 16-byte pieces of an x row sit at
//    piece ^ (row mod 16), so the MFMA operand reads (16 rows, one piece
//    each) and the row writes cover all banks. One barrier per step;
//  - a wave's code words and block scales are loaded three steps ahead, and
//    dequantized one step ahead, between the MFMAs of the step before (2-3 %
//    faster than dequantizing a step's weights ahead of its own MFMAs); dequantization goes through the conflict-free
//    LDS pair table (entry = fp32 code values of both nibbles of a code byte,
//    32 interleaved copies, address built by one v_perm_b32), times the block
//    scale, rounded to the compute dtype in pairs -- the dequantize kernel's
//    weights -- and v_mfma_f32_16x16x32 with x as the A operand;
//  - with one K range the workgroup adds the bias (compute dtype) in fp32,
//    rounds to the output dtype and stores; with S > 1 ranges it stores fp32
//    partial sums [S][M][N] into the caller's workspace and the summing kernel
//    of the split decode path adds the ranges in range order, then the bias.
//    The split depends only on the product's own shape and the CU count, so
//    its bits never depend on what it is grouped with. (The dispatch sends
//    this kernel products of two or more ranges.)
// Out-of-range chunks, rows past N and activation rows m >= M are offsets out
// of the buffer resources' ranges: they read zeros and store nothing.
#include <limits.h>

#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kChunk = 128;                   // codes of one row per step and wave
constexpr int kCopies = 32;                   // interleaved copies of the pair table
constexpr int kTableBytes = 256 * 256;        // 256 entries x 256-byte rows
constexpr int kMaxGroup = 16;
constexpr int kMaxRanges = 8;                 // K ranges, at most (the summing kernel's limit)
constexpr int kWaves = 8;                     // per workgroup (two per SIMD)
constexpr int kWpg = 4;                       // waves per group
// 16-row MFMA tiles per wave: one up to 16 activation rows (64-row blocks, two
// workgroups per CU), else two (128-row blocks, one workgroup per CU)
constexpr int tiles_per_wave(int mt) { return mt == 1 ? 1 : 2; }
constexpr int block_rows(int mt) { return 16 * tiles_per_wave(mt) * kWpg; }
constexpr int kXRowBytes = 2 * kChunk;        // one activation row of a chunk
constexpr int kBufferFlags = 0x00020000;      // word 3 of a raw buffer resource (gfx9)
constexpr uint32_t kOOB = 0x80000000u;        // an offset past every buffer's range

struct TkProblem {
  const char *x;          // activations (compute dtype), row m at m * ldx_bytes
  const uint8_t *packed;  // [N, K / 2] codes
  char *y;                // output, row m at m * ldy_bytes; or the [S][M][N] fp32 partials
  const char *bias;       // [N] compute dtype, or null (one K range only)
  const float *absmax;    // absmax (no double quant) or absmax_scale
  const int8_t *absmax_q;
  const float *absmax_offset;
  int32_t N;
  int32_t wgs;            // workgroups of the problem (blocks x ranges)
  int32_t S, nchs;        // K ranges, and chunks per range
  int32_t log2_bs, log2_bs2;
  uint32_t ldx_bytes, ldy_bytes;
  uint32_t x_bytes, y_bytes;  // ranges of x and of y (or of the partials)
};

struct TkArgs {
  TkProblem p[kMaxGroup];       // problem i takes the workgroups with blockIdx.y == i
  int32_t M, K;
  int32_t out_dtype;            // of the one-range problems (the others store fp32 partials)
  float value[16];
};

// A wave's loads for one chunk of its row tiles.
template <int kNtw>
struct TkCodes {
  uint4 w[kNtw];     // 32 codes of row 16 t + n at k0 + 32 kg
  int32_t q[kNtw];   // int8 block code (double quant)
  float s[kNtw];     // absmax, or the group scale s2
  float mu[kNtw];    // group offset (mean-centred double quant)
};

// 8 codes of one packed word -> 4 packed pairs of the compute type, in k order
// (byte j holds element 2j in its high nibble and 2j + 1 in its low nibble).
template <int CT>
__device__ __forceinline__ uint4 tk_dequant8(uint32_t word, float ap, const char *tbl,
                                             uint32_t lane_base) {
  f32x2 c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // address bytes: [0] lane_base (8 * copy), [1] code byte j, [2..3] zero
    const uint32_t addr = __builtin_amdgcn_perm(word, lane_base, 0x0c0c0000u | ((4u + j) << 8));
    c[j] = *reinterpret_cast<const f32x2 *>(tbl + addr);
  }
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = pack2<CT>(c[j].x * ap, c[j].y * ap);
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// The end of a step: this wave's LDS writes done, then a bare barrier. (A
// workgroup fence would also make every wave wait for all of its loads in
// flight, the prefetches included; the empty asm statements keep the compiler
// from moving memory accesses across the barrier.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int MT, int NST, int DQ, int CT>
__global__ __launch_bounds__(64 * kWaves) void gemv_tk_kernel(TkArgs args) {
  constexpr int kNtw = tiles_per_wave(MT);
  constexpr int kBlockRows = block_rows(MT);
  constexpr int kXRows = 16 * MT;                         // activation rows staged
  constexpr int kStageBytes = 2 * kXRows * kXRowBytes;    // both groups' chunks
  constexpr int kXLoads = kStageBytes / (16 * 64 * kWaves);  // 16-byte loads per thread
  __shared__ __attribute__((aligned(16))) char tbl[kTableBytes];
  __shared__ __attribute__((aligned(16))) char xs[2 * kStageBytes];

  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / kWpg, wig = wave % kWpg;  // group, wave in the group
  const int n = lane & 15, kg = lane >> 4;
  const uint32_t lane_base = 8u * (uint32_t)(lane & (kCopies - 1));
  const int M = args.M, K = args.K;

  // problem (blockIdx.y), row block and K range of this workgroup;
  // workgroups past the problem's own count end at once
  const TkProblem P = args.p[blockIdx.y];
  // every argument needed before the first memory loads, in registers before
  // the early exit, so they come in one batch of loads (otherwise the
  // compiler loads the count first and the rest after the branch: two round
  // trips to the argument block)
  asm volatile("" ::"s"(P.x), "s"(P.packed), "s"(P.absmax), "s"(P.absmax_q), "s"(P.N),
               "s"(P.wgs), "s"(P.S), "s"(P.nchs), "s"(P.log2_bs), "s"(P.log2_bs2),
               "s"(P.ldx_bytes), "s"(P.x_bytes), "s"(args.M), "s"(args.K));
  const int S = P.S;
  const int local = (int)blockIdx.x;
  if (local >= P.wgs) return;
  const int blk = local / S, range = local - blk * S;
  const int row0 = blk * kBlockRows;
  const int rows = P.N - row0 < kBlockRows ? P.N - row0 : kBlockRows;
  const int nch = (K + kChunk - 1) / kChunk;
  const int kc0 = range * P.nchs;
  const int kc1 = kc0 + P.nchs < nch ? kc0 + P.nchs : nch;
  const int steps = (kc1 - kc0 + 1) >> 1;  // chunk pairs
  const uint32_t row_bytes = (uint32_t)K >> 1;

  // ---- buffer resources of the block ----
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(P.packed + (int64_t)row0 * row_bytes), (short)0,
      (int)((uint32_t)rows * row_bytes), kBufferFlags);
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
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.x, (short)0, (int)P.x_bytes, kBufferFlags);

  // Per-thread offsets at step 0; step st adds 2 chunks (256 codes) to every
  // k. A load is in range while its k is below kend (the end of the K range
  // or of the row), and x rows m >= M are never read.
  const int kend = kc1 * kChunk < K ? kc1 * kChunk : K;
  const int log2_bs = P.log2_bs, log2_bs2 = P.log2_bs2;
  const int kw0 = (kc0 + grp) * kChunk + 32 * kg;  // this lane's first code at step 0
  uint32_t wof[kNtw], rk[kNtw];
#pragma unroll
  for (int t = 0; t < kNtw; ++t) {
    const uint32_t r = (uint32_t)(16 * kNtw * wig + 16 * t + n);  // row in the block
    wof[t] = r * row_bytes + ((uint32_t)kw0 >> 1);
    rk[t] = r * (uint32_t)K + (uint32_t)kw0;  // element index in the block at step 0
  }
  int xk[kXLoads];
  uint32_t xof[kXLoads];
#pragma unroll
  for (int j = 0; j < kXLoads; ++j) {
    // flat 16-byte piece f = j * 512 + tid: activation row f / 32, chunk
    // f / 16 % 2 of the step's pair, piece f % 16 of that chunk row
    const int f = j * 64 * kWaves + tid;
    const int m = f >> 5, h = (f >> 4) & 1, pc = f & 15;
    xk[j] = m < M ? (kc0 + h) * kChunk + 8 * pc : INT_MAX / 2;
    xof[j] = (uint32_t)m * P.ldx_bytes + 2u * (uint32_t)((kc0 + h) * kChunk + 8 * pc);
  }

  // code words and scales of this wave's chunk of step st (zeros past the range)
  auto issue_codes = [&](int st) {
    TkCodes<kNtw> u;
    const bool ok = kw0 + 2 * kChunk * st < kend;
#pragma unroll
    for (int t = 0; t < kNtw; ++t) {
      u.w[t] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     wrs, (int)(ok ? wof[t] + (uint32_t)(kChunk * st) : kOOB), 0, 0));
      const uint32_t b = (rk[t] + (uint32_t)(2 * kChunk * st)) >> log2_bs;  // block in the block
      if (DQ == kDqNone) {
        u.q[t] = 1;
        u.mu[t] = 0.0f;
        u.s[t] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(srs, (int)(ok ? 4u * b : kOOB), 0, 0));
      } else {
        const uint32_t g = (blk_in + b) >> log2_bs2;
        u.q[t] = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(qrs, (int)(ok ? b : kOOB), 0, 0);
        u.s[t] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(srs, (int)(ok ? 4u * g : kOOB), 0, 0));
        if (DQ == kDqCentred)
          u.mu[t] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(mrs, (int)(ok ? 4u * g : kOOB), 0, 0));
        else
          u.mu[t] = 0.0f;
      }
    }
    return u;
  };

  auto issue_x = [&](int st, uint4 (&xr)[kXLoads]) {
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const bool ok = xk[j] + 2 * kChunk * st < kend;
      xr[j] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     xrs, (int)(ok ? xof[j] + (uint32_t)(4 * kChunk * st) : kOOB), 0, 0));
    }
  };
  auto store_x = [&](int stage, const uint4 (&xr)[kXLoads]) {
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const int f = j * 64 * kWaves + tid;
      const int m = f >> 5, h = (f >> 4) & 1, pc = f & 15;
      char *dst = xs + stage * kStageBytes + (h * kXRows + m) * kXRowBytes + 16 * (pc ^ (m & 15));
      *reinterpret_cast<uint4 *>(dst) = xr[j];
    }
  };

  f32x4 acc[kNtw][MT];
#pragma unroll
  for (int t = 0; t < kNtw; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The weights of a step, dequantized to MFMA B operands (row tile t, 8-code
  // word s).
  struct TkB {
    uint4 b[kNtw][4];
  };
  auto dequant = [&](const TkCodes<kNtw> &u) {
    TkB r;
#pragma unroll
    for (int t = 0; t < kNtw; ++t) {
      const float ap = scale_from<DQ>(u.q[t], u.s[t], u.mu[t]);
      const uint32_t wd[4] = {u.w[t].x, u.w[t].y, u.w[t].z, u.w[t].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) r.b[t][s] = tk_dequant8<CT>(wd[s], ap, tbl, lane_base);
    }
    return r;
  };
  // One step's MFMAs on weights dequantized during the step before, with the
  // next step's dequantization interleaved: the matrix core runs while the
  // wave's VALU and table reads work on the next weights.
  auto compute = [&](int stage, const TkB &cur, const TkCodes<kNtw> &next, TkB &nb) {
    const char *xb = xs + stage * kStageBytes + grp * kXRows * kXRowBytes;
    float ap[kNtw];
#pragma unroll
    for (int t = 0; t < kNtw; ++t) ap[t] = scale_from<DQ>(next.q[t], next.s[t], next.mu[t]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 xa[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + n;
        xa[mt] = *reinterpret_cast<const uint4 *>(xb + m * kXRowBytes + 16 * ((4 * kg + s) ^ n));
      }
#pragma unroll
      for (int t = 0; t < kNtw; ++t) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[t][mt] = mfma16x16x32<CT>(xa[mt], cur.b[t][s], acc[t][mt]);
        const uint32_t word =
            s == 0 ? next.w[t].x : s == 1 ? next.w[t].y : s == 2 ? next.w[t].z : next.w[t].w;
        nb.b[t][s] = tk_dequant8<CT>(word, ap[t], tbl, lane_base);
      }
    }
  };

  // ---- prologue: x and codes of steps 0 .. kAhead - 1 in flight, x of step 0 staged ----
  // Per step st: x, then the codes, of step st + kAhead are issued; step st
  // is computed; x of step st + 1 goes to its LDS stage. Waiting for that x
  // leaves the loads of the later steps in flight. The steps are unrolled
  // completely (NST of them; the ones past this range's end are skipped): with
  // no loop-carried registers the compiler's waits are exact.
  constexpr int kAhead = 3;
  uint4 xr[NST + kAhead][kXLoads];
  TkCodes<kNtw> ring[NST + kAhead];
#pragma unroll
  for (int st = 0; st < kAhead; ++st) {
    issue_x(st, xr[st]);
    ring[st] = issue_codes(st);
  }
  // The pair table, built while the first loads are in flight: entry
  // e = (value[e >> 4], value[e & 15]) at 256 e + 8 copy. Iteration i of wave
  // w writes entry 16 i + 2 w (lanes 0-31) and the next one (lanes 32-63),
  // copy = lane mod 32; both take value[i] and one of two low values, so
  // every value comes from scalar registers (no staging in LDS, no barrier).
  float lo0 = args.value[2 * wave], lo1 = args.value[2 * wave + 1];
  // (in scalar registers first: a select between the two would otherwise be
  // folded into a vector load indexed by the lane)
  asm volatile("" : "+s"(lo0), "+s"(lo1));
#pragma unroll
  for (int i = 0; i < 256 / (2 * kWaves); ++i) {
    const float hi = args.value[i];
    const float lo = lane < 32 ? lo0 : lo1;
    const int e = 16 * i + 2 * wave + (lane >> 5);
    *reinterpret_cast<f32x2 *>(tbl + 256 * e + 8 * (lane & 31)) = f32x2{hi, lo};
  }

  store_x(0, xr[0]);
  lds_barrier();  // table and stage 0
  TkB bq[NST + 1];
  bq[0] = dequant(ring[0]);

#pragma unroll
  for (int st = 0; st < NST; ++st) {
    if (st >= steps) break;
    if (st + kAhead < NST) {
      issue_x(st + kAhead, xr[st + kAhead]);
      ring[st + kAhead] = issue_codes(st + kAhead);
    }
    // the loads stay ahead of the arithmetic, so the compiler's waits count
    // them as the newest in flight
    __builtin_amdgcn_sched_barrier(0);
    // (past the last step the codes read zeros: that dequantization is unused)
    compute(st & 1, bq[st], ring[st + 1 < NST ? st + 1 : st], bq[st + 1]);
    __builtin_amdgcn_sched_barrier(0);
    if (st + 1 < NST) store_x((st + 1) & 1, xr[st + 1]);  // zeros past the range
    lds_barrier();
  }

  // ---- the two groups' sums meet; group 0 stores ----
  float *red = reinterpret_cast<float *>(xs);  // the x stages are free now
  if (grp == 1) {
#pragma unroll
    for (int t = 0; t < kNtw; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[(((wig * kNtw + t) * MT + mt) * 4 + r) * 64 + lane] = acc[t][mt][r];
  }
  lds_barrier();
  if (grp != 0) return;
  const bool partial = S > 1;
  const int ob = partial || args.out_dtype == kFP32 ? 4 : 2;
  const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.y, (short)0, (int)P.y_bytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.bias, (short)0, (!partial && P.bias != nullptr) ? (int)(2u * (uint32_t)P.N) : 0,
      kBufferFlags);
  // partial sums of range r live at r * M * N floats: row m of it at m * N
  const uint32_t plane = partial ? 4u * (uint32_t)M * (uint32_t)P.N * (uint32_t)range : 0u;
  const uint32_t ld = partial ? 4u * (uint32_t)P.N : P.ldy_bytes;
#pragma unroll
  for (int t = 0; t < kNtw; ++t) {
    // D layout of the 16x16 MFMA: lane l holds rows 4 (l / 16) + r of column l % 16
    const int row = row0 + 16 * kNtw * wig + 16 * t + n;
    const float bias = widen16<CT>(
        __builtin_amdgcn_raw_buffer_load_b16(brs, (int)(2u * (uint32_t)row), 0, 0));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = acc[t][mt][r] + red[(((wig * kNtw + t) * MT + mt) * 4 + r) * 64 + lane];
        const int m = 16 * mt + 4 * kg + r;
        const uint32_t off = (m < M && row < P.N)
                                 ? plane + (uint32_t)m * ld + (uint32_t)row * (uint32_t)ob
                                 : kOOB;
        if (partial || args.out_dtype == kFP32) {
          if (!partial) v += bias;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), yrs, (int)off, 0, 0);
        } else if (args.out_dtype == kFP16) {
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)out_bits<kFP16>(v + bias), yrs, (int)off,
                                                0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)out_bits<kBF16>(v + bias), yrs, (int)off,
                                                0, 0);
        }
      }
  }
}

template <int MT, int NST, int DQ>
hipError_t launch_tk_ct(const TkArgs &args, dim3 grid, int ct, hipStream_t stream) {
  if (ct == kFP16)
    hipLaunchKernelGGL((gemv_tk_kernel<MT, NST, DQ, kFP16>), grid, dim3(64 * kWaves), 0,
                       stream, args);
  else
    hipLaunchKernelGGL((gemv_tk_kernel<MT, NST, DQ, kBF16>), grid, dim3(64 * kWaves), 0,
                       stream, args);
  return hipGetLastError();
}

template <int MT, int NST>
hipError_t launch_tk_dq(const TkArgs &args, dim3 grid, int dq, int ct, hipStream_t stream) {
  if (dq == kDqCentred) return launch_tk_ct<MT, NST, kDqCentred>(args, grid, ct, stream);
  if (dq == kDqSym) return launch_tk_ct<MT, NST, kDqSym>(args, grid, ct, stream);
  return launch_tk_ct<MT, NST, kDqNone>(args, grid, ct, stream);
}

template <int MT>
hipError_t launch_tk_nst(const TkArgs &args, dim3 grid, int nst, int dq, int ct,
                         hipStream_t stream) {
  if (nst == 4) return launch_tk_dq<MT, 4>(args, grid, dq, ct, stream);
  if (nst == 6) return launch_tk_dq<MT, 6>(args, grid, dq, ct, stream);
  return launch_tk_dq<MT, 8>(args, grid, dq, ct, stream);
}

// The K split of a product. A range is at most 16 chunks (8 steps of the
// kernel). Beyond that the product takes as many ranges as keep its
// workgroups (blocks x ranges) within one round on the CUs, but no more than
// make the partial sums (written and read back, 8 S M N bytes) as large as
// the codes (N K / 2 bytes): S <= K / (16 M).
// Rows of a workgroup's block, and workgroups a CU holds at once, by M.
int tk_block_rows(int M) { return block_rows(gemv_row_tiles(M)); }
int tk_wgs_per_cu(int M) { return gemv_row_tiles(M) == 1 ? 2 : 1; }

int tk_ranges(int M, int N, int K) {
  const int nch = (K + kChunk - 1) / kChunk;
  const int smin = (nch + 15) / 16;
  if (smin > kMaxRanges) return 0;
  const int br = tk_block_rows(M);
  const int blocks = (N + br - 1) / br;
  int s = device_cu_count() * tk_wgs_per_cu(M) / (blocks > 0 ? blocks : 1);
  const int cap = K / (16 * M);
  if (s > cap) s = cap;
  if (s > kMaxRanges) s = kMaxRanges;
  if (s < smin) s = smin;
  if (s < 1) s = 1;
  const int nchs = (nch + s - 1) / s;
  return (nch + nchs - 1) / nchs;  // no empty range
}

int tk_chunks_per_range(int M, int N, int K) {
  const int nch = (K + kChunk - 1) / kChunk;
  const int s = tk_ranges(M, N, K);
  return (nch + s - 1) / s;
}

}  // namespace

int gemv_tk_ranges(int M, int N, int K) {
  if (M <= 7 || M > 64 || K <= 0 || N <= 0) return 0;
  const int s = tk_ranges(M, N, K);
  // the partial sums are addressed with 31-bit byte offsets
  if ((int64_t)s * M * N * 4 >= ((int64_t)1 << 31)) return 0;
  return s;
}

size_t gemv_tk_bytes(int M, int N, int K) {
  const int s = gemv_tk_ranges(M, N, K);
  if (s <= 1) return 0;
  return ((size_t)s * (size_t)M * (size_t)N * 4u + 255u) & ~(size_t)255u;
}

bool gemv_tk_enabled() {
  static const bool on = [] {
    const char *v = getenv("NF4_DECODE_TILED");
    return v == nullptr || v[0] != '0';
  }();
  return on;
}

hipError_t launch_gemv_tk(int count, const GemvDesc *descs, int M, int K, int quant_type, int dq,
                          int compute_dtype, int out_dtype, void *workspace, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  if (count > kMaxGroup) return hipErrorInvalidValue;
  const CodeTables &tb = code_tables(quant_type);
  const uint32_t xe = 2u;
  const uint32_t ye = out_dtype == kFP32 ? 4u : 2u;
  TkArgs args;
  args.M = M;
  args.K = K;
  args.out_dtype = out_dtype;
  for (int i = 0; i < 16; ++i) args.value[i] = tb.value[i];
  float *part[kMaxGroup];
  int ranges[kMaxGroup];
  GemvDesc split[kMaxGroup];
  char *ws = static_cast<char *>(workspace);
  int grid = 0, np = 0, ns = 0, steps = 0;
  for (int i = 0; i < count; ++i) {
    const GemvDesc &d = descs[i];
    if (d.N == 0) continue;
    const int S = gemv_tk_ranges(M, d.N, K);
    if (S < 1) return hipErrorInvalidValue;
    TkProblem &q = args.p[np];
    q.x = static_cast<const char *>(d.x);
    q.packed = d.packed;
    q.absmax = dq ? d.sc.absmax_scale : d.sc.absmax;
    q.absmax_q = d.sc.absmax_q;
    q.absmax_offset = d.sc.absmax_offset;
    q.N = d.N;
    q.S = S;
    q.nchs = tk_chunks_per_range(M, d.N, K);
    q.log2_bs = __builtin_ctz((unsigned)d.blocksize);
    q.log2_bs2 = d.sc.log2_bs2;
    q.ldx_bytes = (uint32_t)(d.ldx * xe);
    q.x_bytes = (uint32_t)(((int64_t)(M - 1) * d.ldx + K) * xe);
    if (S > 1) {
      part[ns] = reinterpret_cast<float *>(ws);
      ranges[ns] = S;
      split[ns++] = d;
      ws += gemv_tk_bytes(M, d.N, K);
      q.y = reinterpret_cast<char *>(part[ns - 1]);
      q.bias = nullptr;
      q.ldy_bytes = 4u * (uint32_t)d.N;
      q.y_bytes = 4u * (uint32_t)S * (uint32_t)M * (uint32_t)d.N;
    } else {
      q.y = static_cast<char *>(d.y);
      q.bias = static_cast<const char *>(d.bias);
      q.ldy_bytes = (uint32_t)(d.ldy * ye);
      q.y_bytes = (uint32_t)(((int64_t)(M - 1) * d.ldy + d.N) * ye);
    }
    q.wgs = (d.N + tk_block_rows(M) - 1) / tk_block_rows(M) * S;
    if (q.wgs > grid) grid = q.wgs;
    const int st = (q.nchs + 1) / 2;
    if (st > steps) steps = st;
    ++np;
  }
  if (np == 0) return hipSuccess;
  const int nst = steps <= 4 ? 4 : steps <= 6 ? 6 : 8;
  if (log_on())
    log_msg("decode M=%d K=%d: gemv_tk_kernel (x staged in LDS; first product in %d K "
            "range(s) of %d chunks), %d steps, grid %d x %d%s; %d product(s)",
            M, K, args.p[0].S, args.p[0].nchs, nst, grid, np,
            ns > 0 ? ", then gemv_split_reduce_kernel" : "", np);
  const int mt = gemv_row_tiles(M);
  const dim3 g(grid, np);
  hipError_t e = mt == 4   ? launch_tk_nst<4>(args, g, nst, dq, compute_dtype, stream)
                 : mt == 2 ? launch_tk_nst<2>(args, g, nst, dq, compute_dtype, stream)
                           : launch_tk_nst<1>(args, g, nst, dq, compute_dtype, stream);
  if (e != hipSuccess || ns == 0) return e;
  return launch_gemv_split_sum(ns, split, part, ranges, M, compute_dtype, out_dtype, stream);
}

}  // namespace nf4
