// dequantize.hip -- 4-bit codes back to fp32 or to the bf16 compute dtype.
//
// [usage page icman.com.cn/news/48546, "Configuration": the compute dtype is
//  the precision used after 4-bit dequantization, bf16 preferred; NF4 page,
//  table 数学原理对比, row 缩放机制: value = code value x block scale.]
// w = RN(c[code] * a'), a' = absmax, RN(q * s2) or RN(RN(q * s2) + mu) (the
// double-quant modes); bf16 / fp16 output = RNE(w).
//
// Layout: a wave owns tiles of 1024 consecutive elements and a lane owns
// elements 8l..8l+7 and 512+8l..512+8l+7 of each (one 4-byte code load per
// half; 8 | blocksize, so the 8 share one block scale). Each bf16 store
// instruction then writes 1 KB without gaps. Stores are non-temporal: the
// output is written once and not read back by this kernel, so it should not
// displace other lines from L2. The inputs of a tile (codes, scale parts)
// are loaded two tiles ahead, so their HBM latency overlaps the stores of
// the tiles before. The 16 fp32 code values sit in LDS; a code times 4 is cut
// from the packed word with one bit-field extract and used as the LDS byte
// offset.
#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kThreads = 256;

// One tensor of a launch; tile_begin: its first whole tile in the launch's
// tile numbering.
struct DTensor {
  const uint8_t *packed;
  void *out;
  int64_t n;
  ScaleArgs sc;
  int32_t log2_bs;
  int64_t tile_begin;
};

constexpr int kMaxDGroup = 16;

struct DequantArgs {
  DTensor t[kMaxDGroup];
  int32_t count;
  int64_t total_tiles;  // whole 1024-element tiles over all tensors
  float value[16];
};

// tensor of launch tile lt and the tile's index within it
__device__ __forceinline__ const DTensor &locate_tile(const DequantArgs &args, int64_t lt,
                                                      int64_t &tile) {
  int t = 0;
#pragma unroll 1
  while (t + 1 < args.count && args.t[t + 1].tile_begin <= lt) ++t;
  tile = lt - args.t[t].tile_begin;
  return args.t[t];
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// The raw inputs of one lane for one whole tile: the packed codes of its two
// 8-element pieces and what their block scales are made of.
template <int DQ>
struct TileIn {
  uint32_t word[2];
  float a[2];      // fp32 absmax (no double quant) or absmax_scale
  int32_t q[2];    // int8 absmax code (double quant)
  float mu[2];     // group offset (mean-centred double quant)
};

template <int DQ>
__device__ __forceinline__ TileIn<DQ> load_tile_in(const DequantArgs &args, int64_t lt, int lane) {
  int64_t tile;
  const DTensor &T = locate_tile(args, lt, tile);
  TileIn<DQ> t;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int64_t e0 = tile * 1024 + 512 * half + 8 * lane;
    t.word[half] = *reinterpret_cast<const uint32_t *>(T.packed + e0 / 2);
    const int64_t b = e0 >> T.log2_bs;
    if (DQ) {
      t.q[half] = T.sc.absmax_q[b];
      t.a[half] = T.sc.absmax_scale[b >> T.sc.log2_bs2];
      t.mu[half] = DQ == kDqCentred ? T.sc.absmax_offset[b >> T.sc.log2_bs2] : 0.0f;
    } else {
      t.q[half] = 1;
      t.a[half] = T.sc.absmax[b];
      t.mu[half] = 0.0f;
    }
  }
  return t;
}

// 8 dequantized values of one packed word with block scale ap
__device__ __forceinline__ void decode8(uint32_t word, float ap, const char *tb, float (&w)[8]) {
  // byte j of the word holds element 2j in bits 7..4 and 2j+1 in bits 3..0
  const uint32_t even4 = (word >> 2) & 0x3c3c3c3cu;  // 4 * code(2j) in byte j
  const uint32_t odd4 = (word << 2) & 0x3c3c3c3cu;   // 4 * code(2j+1) in byte j
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[2 * j] = *reinterpret_cast<const float *>(tb + ((even4 >> (8 * j)) & 0xffu)) * ap;
    w[2 * j + 1] = *reinterpret_cast<const float *>(tb + ((odd4 >> (8 * j)) & 0xffu)) * ap;
  }
}

template <int OUT>
__device__ __forceinline__ void store8(void *out, int64_t e0, const float (&w)[8]) {
  if (OUT != kFP32) {
    u32x4 v;
    v.x = pack2<OUT>(w[0], w[1]);
    v.y = pack2<OUT>(w[2], w[3]);
    v.z = pack2<OUT>(w[4], w[5]);
    v.w = pack2<OUT>(w[6], w[7]);
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(out) + e0));
  } else {
    f32x4 v0, v1;
    v0.x = w[0]; v0.y = w[1]; v0.z = w[2]; v0.w = w[3];
    v1.x = w[4]; v1.y = w[5]; v1.z = w[6]; v1.w = w[7];
    f32x4 *o = reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + e0);
    __builtin_nontemporal_store(v0, o);
    __builtin_nontemporal_store(v1, o + 1);
  }
}

template <int OUT, int DQ>
__device__ __forceinline__ void write_tile(const DequantArgs &args, const TileIn<DQ> &in,
                                           int64_t lt, int lane, const char *tb) {
  int64_t t;
  const DTensor &T = locate_tile(args, lt, t);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const float ap = scale_from<DQ>(in.q[half], in.a[half], in.mu[half]);
    float w[8];
    decode8(in.word[half], ap, tb, w);
    store8<OUT>(T.out, t * 1024 + 512 * half + 8 * lane, w);
  }
}

template <int OUT, int DQ>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(DequantArgs args) {
  __shared__ float table[16];
  if (threadIdx.x < 16) table[threadIdx.x] = args.value[threadIdx.x];
  __syncthreads();
  const char *tb = reinterpret_cast<const char *>(table);

  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t nfull = args.total_tiles;  // whole 1024-element tiles

  // whole tiles, two register sets in turn: the inputs of a wave's tile after
  // next are loaded as soon as a set has been decoded, so their latency
  // overlaps the stores of two tiles (indices past the end are clamped: a
  // harmless reload)
  if (wave < nfull) {
    int64_t t = wave;
    auto clampt = [&](int64_t u) { return u < nfull ? u : t; };
    TileIn<DQ> a = load_tile_in<DQ>(args, t, lane);
    TileIn<DQ> b = load_tile_in<DQ>(args, clampt(t + nwaves), lane);
    for (;;) {
      write_tile<OUT, DQ>(args, a, t, lane, tb);
      a = load_tile_in<DQ>(args, clampt(t + 2 * nwaves), lane);
      if (t + nwaves >= nfull) break;
      write_tile<OUT, DQ>(args, b, t + nwaves, lane, tb);
      b = load_tile_in<DQ>(args, clampt(t + 3 * nwaves), lane);
      if (t + 2 * nwaves >= nfull) break;
      t += 2 * nwaves;
    }
  }

  // the ragged last tile of each tensor, element by element where a piece is
  // cut short (tensor i's by wave i mod nwaves)
#pragma unroll 1
  for (int ti = 0; ti < args.count; ++ti) {
    const DTensor &T = args.t[ti];
    if ((T.n & 1023) == 0 || wave != ti % nwaves) continue;
    const int64_t tl = T.n >> 10;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int64_t e0 = tl * 1024 + 512 * half + 8 * lane;
      if (e0 >= T.n) continue;
      const int64_t b = e0 >> T.log2_bs;
      const int64_t g = DQ ? b >> T.sc.log2_bs2 : 0;
      const float ap =
          DQ ? scale_from<DQ>(T.sc.absmax_q[b], T.sc.absmax_scale[g],
                              DQ == kDqCentred ? T.sc.absmax_offset[g] : 0.0f)
             : T.sc.absmax[b];
      const int64_t nbytes = (T.n - e0 + 1) / 2;
      uint32_t word = 0;
      for (int i = 0; i < 4; ++i)
        if (i < nbytes) word |= (uint32_t)T.packed[e0 / 2 + i] << (8 * i);
      float w[8];
      decode8(word, ap, tb, w);
      if (e0 + 8 <= T.n) {
        store8<OUT>(T.out, e0, w);
      } else if (OUT != kFP32) {
        uint16_t *o = reinterpret_cast<uint16_t *>(T.out) + e0;
        for (int i = 0; i < 8 && e0 + i < T.n; ++i) o[i] = (uint16_t)out_bits<OUT>(w[i]);
      } else {
        float *o = reinterpret_cast<float *>(T.out) + e0;
        for (int i = 0; i < 8 && e0 + i < T.n; ++i) o[i] = w[i];
      }
    }
  }
}

template <int OUT, int DQ>
void launch_cfg(dim3 grid, const DequantArgs &args, hipStream_t stream) {
  hipLaunchKernelGGL((dequantize_kernel<OUT, DQ>), grid, dim3(kThreads), 0, stream, args);
}

template <int OUT>
void launch_out(int dq, dim3 grid, const DequantArgs &args, hipStream_t stream) {
  if (dq == kDqCentred) launch_cfg<OUT, kDqCentred>(grid, args, stream);
  else if (dq == kDqSym) launch_cfg<OUT, kDqSym>(grid, args, stream);
  else launch_cfg<OUT, kDqNone>(grid, args, stream);
}

}  // namespace

int dequantize_max_group() { return kMaxDGroup; }

hipError_t launch_dequantize(int count, const DequantDesc *ds, int quant_type, int dq,
                             int out_dtype, hipStream_t stream) {
  if (count > kMaxDGroup) return hipErrorInvalidValue;
  const CodeTables &t = code_tables(quant_type);
  DequantArgs args;
  args.count = 0;
  int64_t tiles = 0;
  for (int i = 0; i < count; ++i) {
    if (ds[i].n == 0) continue;
    DTensor &T = args.t[args.count++];
    T.packed = ds[i].packed;
    T.out = ds[i].out;
    T.n = ds[i].n;
    T.sc = ds[i].sc;
    T.log2_bs = __builtin_ctz((unsigned)ds[i].blocksize);
    T.tile_begin = tiles;
    tiles += T.n >> 10;
  }
  if (args.count == 0) return hipSuccess;
  args.total_tiles = tiles;
  for (int i = 0; i < 16; ++i) args.value[i] = t.value[i];
  // about two tiles of 1024 elements per wave (and a wave for each tensor's
  // ragged tail), at most 64 workgroups per CU: a grouped call over the seven
  // weights of a 7B layer (197632 tiles) ran 9 % faster at this cap than at
  // 16 per CU, and slower again at 96 per CU or without a cap
  int64_t blocks = (tiles + args.count + 4 * 2 - 1) / (4 * 2);
  if (blocks > 16384) blocks = 16384;
  dim3 grid((unsigned)blocks);
  if (out_dtype == kFP16) launch_out<kFP16>(dq, grid, args, stream);
  else if (out_dtype == kFP32) launch_out<kFP32>(dq, grid, args, stream);
  else launch_out<kBF16>(dq, grid, args, stream);
  return hipGetLastError();
}

}  // namespace nf4
