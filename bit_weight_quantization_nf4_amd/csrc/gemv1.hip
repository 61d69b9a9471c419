// gemv1.hip -- decode products with a single activation row (M = 1):
// y_i[j] = sum_k bf16(dequant(W_i))[j, k] * x_i[k], one or several independent
// problems per launch.
//
// [repo page ossradar.top bitsandbytes, release notes 0.50.0: batch-1 4-bit
//  inference uses a 4-bit GEMV; usage page icman.com.cn/news/48546,
//  "Configuration": weights are dequantized to the bf16 compute dtype.]
//
// Design (HBM-bound; every 4-bit weight is read exactly once):
//  - a wave owns whole weight rows. Lane l reads the 16-byte code slices at
//    k = 2048 j + 32 l (j < J = ceil(K / 2048)), so each load instruction
//    streams 1 KB of one row and the lane's activations x[k .. k+31] stay in
//    registers for every row of the problem;
//  - the rows of all problems of the launch are split into contiguous ranges,
//    one per wave, so activations are reloaded only where a range crosses into
//    the next problem; each wave issues the loads of two rows before using
//    them;
//  - dequantization: the same conflict-free LDS pair table as the batched
//    kernel (entry = fp32 code values of both nibbles of a code byte, one copy
//    per bank pair, address built by one v_perm_b32), times the block scale,
//    rounded to bf16 pairs with v_cvt_pk_bf16_f32 -- the dequantize kernel's
//    bf16 weights -- then v_dot2_f32_bf16 with the bf16 activations;
//  - a row ends with a fixed-order DPP reduction across the wave (no atomics),
//    so results are bitwise reproducible.
#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlice = 2048;           // codes of one row per wave-wide load
constexpr int kCopies = 32;            // interleaved copies of the pair table
constexpr int kTableBytes = 256 * 256; // 256 entries x 256-byte rows
constexpr int kMaxGroup = 16;

struct Gemv1Problem {
  const uint16_t *x;
  const uint8_t *packed;
  void *y;
  const float *absmax;
  const int8_t *absmax_q;
  const float *absmax_scale;
  int32_t N, K;
  int32_t log2_bs, log2_bs2;
  int64_t row_begin;  // first row of this problem in the concatenated row list
};

struct Gemv1Args {
  Gemv1Problem p[kMaxGroup];
  int32_t count;
  int64_t total_rows;
  float value[16];
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Sum over the 64 lanes in a fixed order; the total lands in lane 63.
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
  // every lane of a 16-lane row now holds that row's sum; fold the 4 rows
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                            0x142, 0xa, 0xf, false));  // row_bcast:15
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                            0x143, 0xc, 0xf, false));  // row_bcast:31
  return v;
}

// 8 codes of one packed word times the block scale, dotted with 8 bf16
// activations (4 packed pairs), accumulated in fp32.
__device__ __forceinline__ float dot8(uint32_t word, float ap, const uint32_t xp[4],
                                      const char *tbl, uint32_t lane_base, float acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t addr = __builtin_amdgcn_perm(word, lane_base, 0x0c0c0000u | ((4u + j) << 8));
    const f32x2 c = *reinterpret_cast<const f32x2 *>(tbl + addr);
    const uint32_t w2 = pack_bf16x2(c.x * ap, c.y * ap);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w2),
                                          __builtin_bit_cast(bf16x2_t, xp[j]), acc, false);
  }
  return acc;
}

template <int J, bool DQ, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void gemv1_kernel(Gemv1Args args) {
  __shared__ __attribute__((aligned(16))) char tbl[kTableBytes];
  // Pair table, entry e = (value[e >> 4], value[e & 15]) at 256 e + 8 copy.
  // Consecutive lanes write consecutive copies (no bank conflicts); in pass i
  // every entry has e >> 4 == i.
  {
    const float lo = args.value[(threadIdx.x >> 5) & 15];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int idx = threadIdx.x + kThreads * i;  // e = idx / 32, copy = idx % 32
      const f32x2 v = {args.value[i], lo};
      *reinterpret_cast<f32x2 *>(tbl + 256 * (idx >> 5) + 8 * (idx & 31)) = v;
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const uint32_t lane_base = 8u * (uint32_t)(lane & (kCopies - 1));
  const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  const int64_t r_begin = wave * args.total_rows / nwaves;
  const int64_t r_end = (wave + 1) * args.total_rows / nwaves;

  int pi = -1;
  int64_t p_end = 0;  // first row after the current problem
  Gemv1Problem P;
  uint32_t xv[J][16];  // x[2048 j + 32 lane .. +31] as bf16 pairs
  bool sl_ok[J];

  for (int64_t r = r_begin; r < r_end; r += 2) {
    if (r >= p_end) {
      // next problem: the one containing row r
      do {
        ++pi;
      } while (pi + 1 < args.count && args.p[pi + 1].row_begin <= r);
      P = args.p[pi];
      p_end = P.row_begin + P.N;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int k0 = kSlice * j + 32 * lane;
        sl_ok[j] = k0 < P.K;
        const uint4 *src = reinterpret_cast<const uint4 *>(P.x + (sl_ok[j] ? k0 : 0));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = sl_ok[j] ? src[q] : make_uint4(0, 0, 0, 0);
          xv[j][4 * q] = v.x;
          xv[j][4 * q + 1] = v.y;
          xv[j][4 * q + 2] = v.z;
          xv[j][4 * q + 3] = v.w;
        }
      }
    }
    // two rows of this problem (the second may not exist)
    const int64_t rl = r - P.row_begin;
    const bool has2 = r + 1 < r_end && r + 1 < p_end;
    uint4 pw[2][J];
    float sf[2][J];
    int32_t sq[2][J];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t row = rl + (t == 1 && has2 ? 1 : 0);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int64_t e = row * P.K + (sl_ok[j] ? kSlice * j + 32 * lane : 0);
        pw[t][j] = *reinterpret_cast<const uint4 *>(P.packed + e / 2);
        const int64_t b = e >> P.log2_bs;
        if (DQ) {
          sq[t][j] = P.absmax_q[b];
          sf[t][j] = P.absmax_scale[b >> P.log2_bs2];
        } else {
          sq[t][j] = 1;
          sf[t][j] = P.absmax[b];
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float ap = DQ ? (float)sq[t][j] * sf[t][j] : sf[t][j];
        ap = sl_ok[j] ? ap : 0.0f;
        acc = dot8(pw[t][j].x, ap, &xv[j][0], tbl, lane_base, acc);
        acc = dot8(pw[t][j].y, ap, &xv[j][4], tbl, lane_base, acc);
        acc = dot8(pw[t][j].z, ap, &xv[j][8], tbl, lane_base, acc);
        acc = dot8(pw[t][j].w, ap, &xv[j][12], tbl, lane_base, acc);
      }
      const float sum = wave_sum(acc);
      if (lane == 63 && (t == 0 || has2)) {
        const int64_t row = rl + t;
        if (OUT_BF16)
          reinterpret_cast<uint16_t *>(P.y)[row] = (uint16_t)(pack_bf16x2(sum, 0.0f) & 0xffffu);
        else
          reinterpret_cast<float *>(P.y)[row] = sum;
      }
    }
    if (!has2 && r + 1 < r_end) r -= 1;  // the second row was in the next problem
  }
}

template <int J, bool DQ>
hipError_t launch_j(const Gemv1Args &args, int grid, bool out_bf16, hipStream_t stream) {
  if (out_bf16)
    hipLaunchKernelGGL((gemv1_kernel<J, DQ, true>), dim3(grid), dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((gemv1_kernel<J, DQ, false>), dim3(grid), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

template <bool DQ>
hipError_t launch_dq(const Gemv1Args &args, int j, int grid, bool out_bf16, hipStream_t stream) {
  switch (j) {
    case 1: return launch_j<1, DQ>(args, grid, out_bf16, stream);
    case 2: return launch_j<2, DQ>(args, grid, out_bf16, stream);
    case 3: return launch_j<3, DQ>(args, grid, out_bf16, stream);
    case 4: return launch_j<4, DQ>(args, grid, out_bf16, stream);
    case 6: return launch_j<6, DQ>(args, grid, out_bf16, stream);
    default: return launch_j<8, DQ>(args, grid, out_bf16, stream);
  }
}

}  // namespace

int gemv1_max_k() { return 8 * kSlice; }

hipError_t launch_gemv1_grouped(int count, const GemvDesc *descs, int quant_type,
                                bool double_quant, bool out_bf16, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  if (count > kMaxGroup) return hipErrorInvalidValue;
  const CodeTables &t = code_tables(quant_type);
  Gemv1Args args;
  args.count = 0;
  int64_t rows = 0;
  int max_k = 0;
  for (int i = 0; i < count; ++i) {
    const GemvDesc &d = descs[i];
    if (d.N == 0) continue;
    Gemv1Problem &p = args.p[args.count++];
    p.x = d.x;
    p.packed = d.packed;
    p.y = d.y;
    p.absmax = d.sc.absmax;
    p.absmax_q = d.sc.absmax_q;
    p.absmax_scale = d.sc.absmax_scale;
    p.N = d.N;
    p.K = d.K;
    p.log2_bs = __builtin_ctz((unsigned)d.blocksize);
    p.log2_bs2 = d.sc.log2_bs2;
    p.row_begin = rows;
    rows += d.N;
    max_k = d.K > max_k ? d.K : max_k;
  }
  if (args.count == 0) return hipSuccess;
  args.total_rows = rows;
  for (int i = 0; i < 16; ++i) args.value[i] = t.value[i];
  int j = (max_k + kSlice - 1) / kSlice;
  if (j == 5) j = 6;
  if (j == 7) j = 8;
  // at least two rows per wave; two workgroups per CU (LDS-limited)
  const int64_t want = (rows + 2 * kWaves - 1) / (2 * kWaves);
  const int64_t cap = 2 * device_cu_count();
  const int grid = (int)(want < cap ? want : cap);
  return double_quant ? launch_dq<true>(args, j, grid, out_bf16, stream)
                      : launch_dq<false>(args, j, grid, out_bf16, stream);
}

}  // namespace nf4
