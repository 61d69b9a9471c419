// nf4_common.h -- types and small helpers shared by the gfx950 kernels and the
// host dispatch code of libnf4. Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kQuantNF4 = 0;
constexpr int kQuantFP4 = 1;

// Element types (the values of nf4_dtype).
constexpr int kBF16 = 0;
constexpr int kFP32 = 1;
constexpr int kFP16 = 2;

// Double-quant modes (the values of nf4_double_quant_mode).
constexpr int kDqNone = 0;
constexpr int kDqSym = 1;
constexpr int kDqCentred = 2;

// Number of cells of the quantize lookup: cell i holds every normalised value
// s in [-1, 1] with floor(round-to-nearest(128 s + 128) / 8) == i.
constexpr int kCells = 33;

// Per-type constant tables, built once on the host and passed to kernels by
// value (they live in the kernel-argument segment).
struct CodeTables {
  // fp32 code value for each 4-bit code (the dequantization table)
  float value[16];
  // quantize lookup: within cell i the code is (s > cell_thr[i]) ? hi : lo;
  // cell_codes[i] holds lo, hi in bytes 0, 1 and lo << 4, hi << 4 in bytes 2, 3
  float cell_thr[kCells];
  uint32_t cell_codes[kCells];
};

// Effective-scale source of one quantized tensor as the kernels read it.
struct ScaleArgs {
  const float *absmax;       // [nb] when double quant is off
  const int8_t *absmax_q;    // [nb] with double quant
  const float *absmax_scale; // [ceil(nb / bs2)] with double quant
  const float *absmax_offset;// [ceil(nb / bs2)] in the mean-centred mode
  int32_t log2_bs2;          // log2(blocksize2)
  int32_t double_quant;      // kDqNone, kDqSym or kDqCentred
};

// a' from the raw parts of a block scale: the fp32 absmax (kDqNone), RN(q s2)
// (kDqSym) or RN(RN(q s2) + mu) (kDqCentred). q is the int8 code as an int;
// the build keeps multiply and add separate (no contraction).
template <int DQ>
__device__ __forceinline__ float scale_from(int32_t q, float s2_or_absmax, float mu) {
  if (DQ == kDqNone) return s2_or_absmax;
  const float t = (float)q * s2_or_absmax;
  if (DQ == kDqSym) return t;
  return t + mu;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}


// Bit-field extract of 8 bits at a constant offset as one v_bfe_u32 (the
// compiler otherwise splits a chain of extracts from one pre-shifted word
// into a shift and a mask per field).
template <int OFF>
__device__ __forceinline__ uint32_t bfe8(uint32_t v) {
  uint32_t r;
  asm("v_bfe_u32 %0, %1, %2, 8" : "=v"(r) : "v"(v), "i"(OFF));
  return r;
}

// Two fp32 -> packed bf16 pair with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Two fp32 -> packed fp16 pair, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  f16x2 h = __builtin_convertvector(f, f16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// Two fp32 -> a packed pair of the 16-bit compute type CT (kBF16 / kFP16).
template <int CT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (CT == kFP16) return pack_f16x2(lo, hi);
  else return pack_bf16x2(lo, hi);
}

// A 16-bit pattern of type CT widened (exactly) to fp32.
template <int CT>
__device__ __forceinline__ float widen16(uint32_t bits16) {
  if constexpr (CT == kFP16) {
    const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
    return (float)h;
  } else {
    return __uint_as_float(bits16 << 16);
  }
}

// The 16 low bits of the OUT-type rounding of v (kBF16 / kFP16), or its fp32
// bits (kFP32).
template <int OUT>
__device__ __forceinline__ uint32_t out_bits(float v) {
  if constexpr (OUT == kFP32) return __float_as_uint(v);
  else return pack2<OUT>(v, 0.0f) & 0xffffu;
}

// 16x16x32 matrix-core step in compute type CT: acc += A(16x32) B(32x16), the
// operands as 8 packed 16-bit values per lane.
template <int CT>
__device__ __forceinline__ f32x4 mfma16x16x32(uint4 a, uint4 b, f32x4 acc) {
  if constexpr (CT == kFP16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

}  // namespace nf4
