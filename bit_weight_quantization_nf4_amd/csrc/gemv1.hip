// gemv1.hip -- decode products with a single activation row (M = 1):
// y_i[j] = sum_k bf16(dequant(W_i))[j, k] * x_i[k], one or several independent
// problems per launch.
//
// [repo page ossradar.top bitsandbytes, release notes 0.50.0: batch-1 4-bit
//  inference uses a 4-bit GEMV; usage page icman.com.cn/news/48546,
//  "Configuration": weights are dequantized to the bf16 compute dtype.]
//
// Design (HBM-bound; every 4-bit weight is read exactly once):
//  - a wave owns whole weight rows. Lane l reads the 32 code bytes at
//    k = 4096 j + 64 l (j < J = ceil(K / 4096)) as two 16-byte loads, so each
//    load instruction streams 1 KB of one row, one block scale per lane covers
//    them (two at blocksize 32), and the lane's activations x[k .. k+63] stay
//    in registers for every row of the problem;
//  - the workgroups of the launch (8 waves each) are split among its problems
//    in proportion to their rows; a workgroup takes a contiguous range of one
//    problem's rows and each of its waves a contiguous share of that, so
//    every wave streams whole rows in address order. A wave keeps the loads
//    of the next row in flight while it computes the current one;
//  - x is fetched once per workgroup (16 bytes per thread per 4096-code
//    slice) and handed to the waves through LDS, instead of every wave
//    fetching all of it: the start-up traffic of a wave is its first rows,
//    not the activation vector;
//  - start-up: a workgroup finds its problem with one batch of scalar loads
//    and issues its activation and first-row loads before it builds the
//    table, so their latency overlaps the table build and the barrier;
//  - balance: a wave's issue priority falls as its rows get done, so the
//    waves sharing a SIMD finish together instead of oldest-first;
//  - dequantization: the same conflict-free LDS pair table as the batched
//    kernel (entry = fp32 code values of both nibbles of a code byte, one copy
//    per bank pair, address built by one v_perm_b32), times the block scale,
//    rounded to bf16 pairs with v_cvt_pk_bf16_f32 -- the dequantize kernel's
//    bf16 weights -- then v_dot2_f32_bf16 with the bf16 activations. This
//    arithmetic (five instructions, about 12 SIMD cycles, per code byte, i.e.
//    per two weights) keeps the SIMDs busy most of the main loop: it and the
//    clock the chip holds under it set about half of the kernel's pace;
//  - a row ends with a fixed-order reduction across the wave (DPP within
//    16-lane rows, then the 16- and 32-lane swaps; no atomics), so results are
//    bitwise reproducible;
//  - an optional bf16 bias per output row (nf4_linear) is loaded with the
//    row's codes and added to the row's fp32 sum.
#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kSlice = 4096;           // codes of one row per slice (64 per lane)
constexpr int kCopies = 32;            // interleaved copies of the pair table
constexpr int kTableBytes = 256 * 256; // 256 entries x 256-byte rows
constexpr int kMaxGroup = 16;
// Word 3 of a raw (untyped, unswizzled) buffer resource on gfx9.
constexpr int kBufferFlags = 0x00020000;

struct Gemv1Problem {
  const uint16_t *x;
  const uint8_t *packed;
  void *y;
  const uint16_t *bias;  // [N] bf16 or null
  const float *absmax;
  const int8_t *absmax_q;
  const float *absmax_scale;
  int32_t N, K;
  int32_t log2_bs, log2_bs2;
};

// The fields every wave reads first (code values, wave ranges, row counts)
// lead the argument block, so one batch of scalar loads brings them all.
struct Gemv1Args {
  float value[16];
  // problem i (of N = rows[i] rows) is served by workgroups wg_begin[i] ..
  // wg_begin[i] + wgs[i] - 1; unused entries have wgs[i] = 0
  int32_t wg_begin[kMaxGroup];
  int32_t wgs[kMaxGroup];
  int32_t rows[kMaxGroup];
  Gemv1Problem p[kMaxGroup];
  int32_t count;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Sum over the 64 lanes in a fixed order; the total lands in lanes 48..63.
__device__ __forceinline__ float wave_sum(float v) {
  // within quads, then 8- and 16-lane rows (xor-style partners via DPP)
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                            0xb1, 0xf, 0xf, false));  // quad_perm 1,0,3,2
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                            0x4e, 0xf, 0xf, false));  // quad_perm 2,3,0,1
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                            0x141, 0xf, 0xf, false));  // row_half_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                            0x140, 0xf, 0xf, false));  // row_mirror
  // every lane of a 16-lane row now holds that row's sum r0..r3; a 16-lane
  // swap gives rows 1 and 3 the sums of rows 0 and 2, a 32-lane swap gives
  // lanes 32..63 those of lanes 0..31: lanes 48..63 end with (r3 + r2) + (r1 + r0)
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  v += __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_permlane16_swap(u, u, false, false)[0]);
  const uint32_t t = __builtin_bit_cast(uint32_t, v);
  v += __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_permlane32_swap(t, t, false, false)[0]);
  return v;
}

// 32 codes (one 16-byte piece) times the block scale, dotted with 32 bf16
// activations (16 packed pairs): all 16 table reads are issued before the
// arithmetic, and two accumulators alternate, so table-read latency and the
// accumulation chain overlap with other work of the wave.
__device__ __forceinline__ void dot32(const uint4 &pw, float ap, const uint32_t xp[16],
                                      const char *tbl, uint32_t lane_base, float &acc0,
                                      float &acc1) {
  const uint32_t wd[4] = {pw.x, pw.y, pw.z, pw.w};
  f32x2 c[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t addr =
        __builtin_amdgcn_perm(wd[i >> 2], lane_base, 0x0c0c0000u | ((4u + (i & 3)) << 8));
    c[i] = *reinterpret_cast<const f32x2 *>(tbl + addr);
  }
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const uint32_t w0 = pack_bf16x2(c[i].x * ap, c[i].y * ap);
    const uint32_t w1 = pack_bf16x2(c[i + 1].x * ap, c[i + 1].y * ap);
    acc0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w0),
                                           __builtin_bit_cast(bf16x2_t, xp[i]), acc0, false);
    acc1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w1),
                                           __builtin_bit_cast(bf16x2_t, xp[i + 1]), acc1, false);
  }
}

// Loads of one weight row: per slice, 64 codes (two 16-byte pieces) per lane
// plus the raw block scales (one block per lane, two when blocksize is 32).
template <int J, bool BS32>
struct RowLoads {
  uint4 pw[J][2];
  float sf[J][BS32 ? 2 : 1];
  int32_t sq[J][BS32 ? 2 : 1];
  uint32_t bias;  // bf16 bits of the row's bias (0 without one)
};

// Waves per SIMD the register budget is sized for: x for J slices lives in
// registers, so longer rows trade occupancy for registers.
template <int J>
constexpr int waves_per_simd() { return J == 1 ? 4 : 2; }

// A workgroup is 8 waves: two share a CU when a SIMD holds 4 waves, one
// fills it when it holds 2.
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
template <int J>
constexpr int wgs_per_cu() { return 4 * waves_per_simd<J>() / kWaves; }

template <int J, int NBUF, bool DQ, bool BS32, bool OUT_BF16>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(waves_per_simd<J>(), waves_per_simd<J>())))
void gemv1_kernel(Gemv1Args args) {
  __shared__ __attribute__((aligned(16))) char tbl[kTableBytes];
  // x of the workgroup's problem, slice j at 8 KB j; lane l's 16-byte piece
  // q of a slice sits at index 64 q + (l + 2 q) mod 64: the 16 lanes of a
  // piece read (same q) and the 16 threads of a store (8 q's, 2 l's) each
  // cover all 16 bank groups, so neither conflicts
  __shared__ uint4 xs[J * 512];

  const int lane = threadIdx.x & 63;
  const uint32_t lane_base = 8u * (uint32_t)(lane & (kCopies - 1));
  // wave index made explicitly uniform, so row bookkeeping stays scalar
  const int wave_in_block = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));

  // Each problem has its own set of waves, each with a contiguous range of
  // that problem's rows. The wave finds its problem with independent scalar
  // loads of the wave ranges (no chain of dependent argument loads), so
  // every wave issues its first memory loads equally early. A wave never
  // switches problems, so its prefetch never restarts. A wave without rows
  // (small launches) still builds its share of the table.
  int wb[kMaxGroup], wn[kMaxGroup], wr[kMaxGroup];
  float val[16];
#pragma unroll
  for (int i = 0; i < kMaxGroup; ++i) {
    wb[i] = args.wg_begin[i];
    wn[i] = args.wgs[i];
    wr[i] = args.rows[i];
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) val[i] = args.value[i];
  // keep these loads in the first batch, ahead of the wave's vector loads
  __builtin_amdgcn_sched_barrier(0);
  int pi = -1, g = 0, ng = 1, nrows = 0;
#pragma unroll
  for (int i = 0; i < kMaxGroup; ++i) {
    const int d = (int)blockIdx.x - wb[i];
    const bool hit = d >= 0 && d < wn[i];
    pi = hit ? i : pi;
    g = hit ? d : g;
    ng = hit ? wn[i] : ng;
    nrows = hit ? wr[i] : nrows;
  }
  {
    const bool has_problem = pi >= 0;
    if (!has_problem) pi = 0;
    // rows [a N / b, (a + 1) N / b) in 32-bit pieces: a N / b = a q + a r / b
    // with N = q b + r, a r < b^2
    auto split = [](uint32_t n, uint32_t a, uint32_t b) {
      const uint32_t q = n / b, r = n % b;
      return a * q + (a * r) / b;
    };
    // the workgroup's rows of the problem, then this wave's contiguous share
    const uint32_t g0 = split((uint32_t)nrows, (uint32_t)g, (uint32_t)ng);
    const uint32_t g1 = split((uint32_t)nrows, (uint32_t)g + 1, (uint32_t)ng);
    const uint32_t w0 = g0 + split(g1 - g0, (uint32_t)wave_in_block, kWaves);
    const uint32_t w1 = g0 + split(g1 - g0, (uint32_t)wave_in_block + 1, kWaves);
    // row counters in 32 bits (a problem has fewer than 2^31 rows): their
    // compares stay scalar
    const int32_t first = (int32_t)w0;
    int32_t cnt = (int32_t)(w1 - w0);
    if (!has_problem) cnt = 0;
    const bool active = cnt > 0;
    const uint16_t *x = args.p[pi].x;
    const uint8_t *packed = args.p[pi].packed;
    const float *absmax = args.p[pi].absmax;
    const int8_t *absmax_q = args.p[pi].absmax_q;
    const float *absmax_scale = args.p[pi].absmax_scale;
    void *y = args.p[pi].y;
    const uint16_t *bias = args.p[pi].bias;
    const bool has_bias = bias != nullptr;
    const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)bias, (short)0, has_bias ? (int)(2u * (uint32_t)nrows) : 0, kBufferFlags);
    const int K = args.p[pi].K;
    const int log2_bs = args.p[pi].log2_bs, log2_bs2 = args.p[pi].log2_bs2;
    const uint32_t row_bytes = (uint32_t)K >> 1;
    const uint32_t row_blocks = (uint32_t)K >> log2_bs;
    // blocksize 32: a lane's 64 codes span two blocks (only in the BS32
    // variant, which a launch uses when any of its problems has bs 32)
    const bool two_blocks = BS32 && log2_bs == 5;

    // Slice j, lane l: codes k0 .. k0+63 with k0 = 4096 j + 64 l, as two
    // 32-code pieces (each wholly inside or outside K, since K % 32 == 0).
    // An absent piece reads zeros and gets block scale 0.
    bool ok[J][2];
    uint32_t voff[J], kb[J], kb2[J];  // kb2: the lane's second block (bs 32), else kb
    uint32_t xv[J][32];         // x[k0 .. k0+63] as bf16 pairs
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int k0 = kSlice * j + 64 * lane;
      ok[j][0] = k0 < K;
      ok[j][1] = k0 + 32 < K;
      voff[j] = ok[j][0] ? (uint32_t)k0 >> 1 : 0x80000000u;  // past the row: reads zeros
      kb[j] = ok[j][0] ? (uint32_t)k0 >> log2_bs : 0u;
      kb2[j] = (two_blocks && ok[j][1]) ? kb[j] + 1 : kb[j];
    }
    // x, once for the workgroup: thread t fetches bytes 16 t .. 16 t + 15 of
    // every 8 KB slice (past K the buffer returns zeros, without a branch)
    uint4 xg[J];
    {
      const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
          (void *)x, (short)0, (int)(2u * (uint32_t)K), kBufferFlags);
#pragma unroll
      for (int j = 0; j < J; ++j)
        xg[j] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)(16 * threadIdx.x + 8192 * j), 0, 0));
    }

    // Row loads go through buffer resources whose base is the (wave-uniform)
    // row start: lane offsets stay 32-bit, no 64-bit vector addresses are
    // formed, and an out-of-range offset returns zeros without an access.
    const uint32_t kAll = 0xffffffffu;
    auto load_row = [&](int64_t rl) {
      RowLoads<J, BS32> L;
      const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(packed + (uint64_t)rl * row_bytes), (short)0, (int)row_bytes, kBufferFlags);
      // first block of the row, and its group split into a group base and
      // the block's place inside that group (64-bit safe)
      const uint64_t rb = (uint64_t)rl * row_blocks;
      const uint64_t gbase = rb >> log2_bs2;
      const uint32_t rb_in = (uint32_t)(rb & (((uint64_t)1 << log2_bs2) - 1));
      // scales first: a wait for a row's scale then leaves its codes in flight
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if (DQ) {
          const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
              (void *)(absmax_q + rb), (short)0, (int)kAll, kBufferFlags);
          L.sq[j][0] = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(qrs, (int)kb[j], 0, 0);
          if constexpr (BS32)  // kb2 == kb unless a second block exists
            L.sq[j][1] = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(qrs, (int)kb2[j], 0, 0);
          // group scale: a per-lane load (lanes of one group share a cache
          // line); no branch, so the waits of later rows stay exact
          const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
              (void *)(absmax_scale + gbase), (short)0, (int)kAll, kBufferFlags);
          L.sf[j][0] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(
                         srs, (int)(((rb_in + kb[j]) >> log2_bs2) << 2), 0, 0));
          if constexpr (BS32)
            L.sf[j][1] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(
                           srs, (int)(((rb_in + kb2[j]) >> log2_bs2) << 2), 0, 0));
        } else {
          const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
              (void *)(absmax + rb), (short)0, (int)kAll, kBufferFlags);
          L.sq[j][0] = 1;
          L.sf[j][0] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(ars, (int)(kb[j] << 2), 0, 0));
          if constexpr (BS32) {
            L.sq[j][1] = 1;
            L.sf[j][1] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(ars, (int)(kb2[j] << 2), 0, 0));
          }
        }
      }
#pragma unroll
      for (int j = 0; j < J; ++j) {
        L.pw[j][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   prs, (int)voff[j], 0, 0));
        // (all of the offset in the range-checked vector part: a piece past
        // the row reads zeros)
        L.pw[j][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   prs, (int)(voff[j] + 16u), 0, 0));
      }
      // the row's bias (a uniform address; no bias: an empty range, reads 0)
      L.bias = __builtin_amdgcn_raw_buffer_load_b16(brs, (int)(2u * (uint32_t)rl), 0, 0);
      // keep the scheduler from hoisting the previous row's arithmetic (and
      // its waits) above these loads
      __builtin_amdgcn_sched_barrier(0);
      return L;
    };

    constexpr uint32_t kOutBytes = OUT_BF16 ? 2u : 4u;
    auto compute_row = [&](const RowLoads<J, BS32> &L, int64_t r) {
      float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int si = BS32 ? p : 0;
          float ap = DQ ? (float)L.sq[j][si] * L.sf[j][si] : L.sf[j][si];
          ap = ok[j][p] ? ap : 0.0f;
          dot32(L.pw[j][p], ap, &xv[j][16 * p], tbl, lane_base, acc0, acc1);
        }
      }
      float sum = wave_sum(acc0 + acc1);
      if (has_bias) sum += bf16_bits_to_f32(L.bias);
      // Lane 63 holds the total. Every lane issues the store (no branch, so
      // the compiler counts it and its waits for later rows stay exact); the
      // buffer is the one output element, and the other lanes' offsets lie
      // past it, so their stores are dropped.
      const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
          (void *)((char *)y + (uint64_t)r * kOutBytes), (short)0, (int)kOutBytes, kBufferFlags);
      const uint32_t yoff = lane == 63 ? 0u : 0x80000000u;
      if (OUT_BF16)
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pack_bf16x2(sum, 0.0f) & 0xffffu), yrs,
                                              (int)yoff, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sum), yrs, (int)yoff,
                                              0, 0);
    };

    // NBUF row buffers in turn: the loads of the next NBUF-1 rows are in
    // flight while the current row computes (per SIMD the arithmetic of a row
    // takes about as long as its bytes take to arrive). An iteration handles
    // NBUF rows with one straight-line body; every prefetch is unconditional
    // (clamped to the last row), so the wait before a row counts only that
    // row's own loads.
    // (a wave without rows prefetches a valid row, first, and computes none)
    const int32_t last = cnt > 0 ? cnt - 1 : 0;
    auto row_at = [&](int32_t i) { return (int64_t)(first + (i < last ? i : last)); };
    RowLoads<J, BS32> buf[NBUF];
#pragma unroll
    for (int b = 0; b + 1 < NBUF; ++b) buf[b] = load_row(row_at(b));

    // Pair table, entry e = (value[e >> 4], value[e & 15]) at 256 e + 8 copy,
    // built while the first loads are in flight, two copies per 16-byte
    // store; consecutive threads write consecutive copies (no bank
    // conflicts). Iteration k of wave w writes entries 32 k + 4 w + lane / 16:
    // their high value, value[2 k + w / 4], is the wave's, and their low one,
    // value[4 (w mod 4) + lane / 16], one of four the wave picks in scalar
    // registers, so every value comes from the argument block's scalars (no
    // staging in LDS, no barrier for it; a lane-dependent index into the
    // argument copy would move all 16 values into vector registers).
    {
      const int w = wave_in_block;
      float c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = val[i];
#pragma unroll
        for (int q = 1; q < 4; ++q) v = (w & 3) == q ? val[4 * q + i] : v;
        // (made explicitly uniform, so the lane select below cannot be folded
        // into a load indexed by the lane)
        c[i] = __builtin_bit_cast(float,
                                  __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
      }
      const int l16 = lane >> 4;
      const float lo = l16 == 0 ? c[0] : l16 == 1 ? c[1] : l16 == 2 ? c[2] : c[3];
#pragma unroll
      for (int k = 0; k < 256 * kCopies / 2 / kThreads; ++k) {
        const float hi = (w >> 2) ? val[2 * k + 1] : val[2 * k];
        const int e = 32 * k + 4 * w + l16;
        const f32x4 v = {hi, lo, hi, lo};
        *reinterpret_cast<f32x4 *>(tbl + 256 * e + 16 * (lane % (kCopies / 2))) = v;
      }
    }
    // piece t of a slice belongs to lane t / 8, as its piece t % 8
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int q = threadIdx.x % 8, l = threadIdx.x / 8;
      xs[512 * j + 64 * q + ((l + 2 * q) & 63)] = xg[j];
    }
    __syncthreads();
    if (!active) return;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint4 v = xs[512 * j + 64 * q + ((lane + 2 * q) & 63)];
        xv[j][4 * q] = v.x;
        xv[j][4 * q + 1] = v.y;
        xv[j][4 * q + 2] = v.z;
        xv[j][4 * q + 3] = v.w;
      }
    // Issue priority falls as the wave's rows get done (four steps): a SIMD
    // otherwise issues for its oldest wave first, so its waves finish one
    // after another and the last runs alone, waiting on memory; with waves
    // that are behind going first they finish together (and late starters
    // catch up).
    const int32_t q1 = cnt / 4, q2 = cnt / 2, q3 = (3 * cnt) / 4;
    for (int32_t i = 0; i < cnt; i += NBUF) {
      if (i < q1) __builtin_amdgcn_s_setprio(3);
      else if (i < q2) __builtin_amdgcn_s_setprio(2);
      else if (i < q3) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int b = 0; b < NBUF; ++b) {
        buf[(b + NBUF - 1) % NBUF] = load_row(row_at(i + b + NBUF - 1));
        // rows past the range are skipped (a uniform branch); written this
        // way, the compiler's waits before each row count exactly the loads
        // of the rows still ahead
        if (i + b <= last) compute_row(buf[b], row_at(i + b));
      }
    }
  }
}

// Splits the workgroups of the launch among the problems in proportion to
// their rows (each gets at least one, and no more than it has rows for one
// per wave); returns the grid size.
template <int J>
int assign_wgs(Gemv1Args &args, int64_t rows) {
  // at least two rows per wave; as many workgroups as fit on the chip at once
  const int64_t want = (rows + 2 * kWaves - 1) / (2 * kWaves);
  const int64_t cap = (int64_t)device_cu_count() * wgs_per_cu<J>();
  int64_t grid = want < cap ? want : cap;
  grid = grid > args.count ? grid : args.count;
  const int64_t spare = grid - args.count;  // beyond the one workgroup each
  int wb = 0;
  for (int i = 0; i < args.count; ++i) {
    const Gemv1Problem &p = args.p[i];
    const int64_t most = (p.N + kWaves - 1) / kWaves;
    int64_t n = 1 + p.N * spare / rows;
    n = n > most ? most : n;
    args.wg_begin[i] = wb;
    args.wgs[i] = (int)n;
    args.rows[i] = p.N;
    wb += (int)n;
  }
  return wb;
}

template <int J, bool DQ, bool BS32>
hipError_t launch_j(Gemv1Args &args, int64_t rows, bool out_bf16, hipStream_t stream) {
  // one row in flight while one computes: deeper prefetch measured no faster
  // (the row's arithmetic, not memory latency, sets the pace)
  constexpr int NBUF = 2;
  const int grid = assign_wgs<J>(args, rows);
  if (out_bf16)
    hipLaunchKernelGGL((gemv1_kernel<J, NBUF, DQ, BS32, true>), dim3(grid), dim3(kThreads), 0,
                       stream, args);
  else
    hipLaunchKernelGGL((gemv1_kernel<J, NBUF, DQ, BS32, false>), dim3(grid), dim3(kThreads), 0,
                       stream, args);
  return hipGetLastError();
}

template <bool DQ, bool BS32>
hipError_t launch_dq(Gemv1Args &args, int64_t rows, int j, bool out_bf16, hipStream_t stream) {
  switch (j) {
    case 1: return launch_j<1, DQ, BS32>(args, rows, out_bf16, stream);
    case 2: return launch_j<2, DQ, BS32>(args, rows, out_bf16, stream);
    case 3: return launch_j<3, DQ, BS32>(args, rows, out_bf16, stream);
    default:
      // four slices at blocksize 32 would need more than 256 registers: those
      // products take the MFMA decode kernel instead (never reached)
      if constexpr (BS32) return hipErrorInvalidValue;
      else return launch_j<4, DQ, BS32>(args, rows, out_bf16, stream);
  }
}

}  // namespace

int gemv1_max_k(int blocksize) { return (blocksize == 32 ? 3 : 4) * kSlice; }

hipError_t launch_gemv1_grouped(int count, const GemvDesc *descs, int quant_type,
                                bool double_quant, bool out_bf16, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  if (count > kMaxGroup) return hipErrorInvalidValue;
  // A launch takes the blocksize-32 variant when any of its products has
  // blocksize 32, and that variant stops at three slices: a group that also
  // holds longer products of other blocksizes goes out as two launches (a
  // product's result does not depend on the launch it is in).
  bool any32 = false, long_other = false;
  for (int i = 0; i < count; ++i) {
    any32 = any32 || descs[i].blocksize == 32;
    long_other = long_other || (descs[i].blocksize != 32 && descs[i].K > 3 * kSlice);
  }
  if (any32 && long_other) {
    GemvDesc a[kMaxGroup], b[kMaxGroup];
    int na = 0, nb = 0;
    for (int i = 0; i < count; ++i) {
      if (descs[i].blocksize == 32) a[na++] = descs[i];
      else b[nb++] = descs[i];
    }
    const hipError_t e = launch_gemv1_grouped(na, a, quant_type, double_quant, out_bf16, stream);
    if (e != hipSuccess) return e;
    return launch_gemv1_grouped(nb, b, quant_type, double_quant, out_bf16, stream);
  }
  const CodeTables &t = code_tables(quant_type);
  Gemv1Args args;
  args.count = 0;
  for (int i = 0; i < kMaxGroup; ++i) {
    args.wg_begin[i] = 0;
    args.wgs[i] = 0;
    args.rows[i] = 0;
  }
  int64_t rows = 0;
  int max_k = 0;
  bool bs32 = false;
  for (int i = 0; i < count; ++i) {
    const GemvDesc &d = descs[i];
    if (d.N == 0) continue;
    Gemv1Problem &p = args.p[args.count++];
    p.x = static_cast<const uint16_t *>(d.x);
    p.packed = d.packed;
    p.y = d.y;
    p.bias = static_cast<const uint16_t *>(d.bias);
    p.absmax = d.sc.absmax;
    p.absmax_q = d.sc.absmax_q;
    p.absmax_scale = d.sc.absmax_scale;
    p.N = d.N;
    p.K = d.K;
    p.log2_bs = __builtin_ctz((unsigned)d.blocksize);
    p.log2_bs2 = d.sc.log2_bs2;
    rows += d.N;
    max_k = d.K > max_k ? d.K : max_k;
    bs32 = bs32 || d.blocksize == 32;
  }
  if (args.count == 0) return hipSuccess;
  for (int i = 0; i < 16; ++i) args.value[i] = t.value[i];
  const int j = (max_k + kSlice - 1) / kSlice;
  if (bs32)
    return double_quant ? launch_dq<true, true>(args, rows, j, out_bf16, stream)
                        : launch_dq<false, true>(args, rows, j, out_bf16, stream);
  return double_quant ? launch_dq<true, false>(args, rows, j, out_bf16, stream)
                      : launch_dq<false, false>(args, rows, j, out_bf16, stream);
}

}  // namespace nf4
