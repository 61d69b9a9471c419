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
  const float *absmax;      // [nb] when double quant is off
  const int8_t *absmax_q;   // [nb] when double quant is on
  const float *absmax_scale;// [ceil(nb / bs2)]
  int32_t log2_bs2;         // log2(blocksize2)
  int32_t double_quant;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// a' of block b: the fp32 absmax, or RN(float(q) * s2) with double quant.
__device__ __forceinline__ float block_scale(const ScaleArgs &sc, int64_t b) {
  if (sc.double_quant) {
    float q = (float)sc.absmax_q[b];
    return q * sc.absmax_scale[b >> sc.log2_bs2];
  }
  return sc.absmax[b];
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

}  // namespace nf4
