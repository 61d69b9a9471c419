// nf4_tables.hip -- host derivation of the NF4/FP4 code tables and of the
// quantize kernel's cell lookup. Runs once per process.
//
// NF4 [NF4 page, CSDN "bitsandbytes 是一个用于高效量化和加载大型语言模型（LLM）的
// 开源库", table 数学原理对比, row 数值表示]: sixteen values from a standard normal
// truncated at delta, normalised to [-1, 1] and containing an exact 0. Levels:
// seven equal probability steps between 1/2 and delta on the negative side,
// eight on the positive side; delta = 929/960 (the page prints the resulting
// -1, -0.697, -0.525, ..., 0, ..., +1). Quantiles are found here by Newton's
// method on the upper tail in long double precision.
//
// FP4 [NF4 page, notes 补充说明: fp4 is a float like E2M1]: the E2M1 value set
// {0, 0.5, 1, 1.5, 2, 3, 4, 6} divided by 6, nibble = sign<<3 | exponent<<1 |
// mantissa.
#include <math.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "nf4_internal.h"

namespace nf4 {
namespace {

// z >= 0 with P(Z > z) = q, 0 < q <= 1/2. The upper tail is convex and
// decreasing on z >= 0, so Newton's iteration from z = 0 increases
// monotonically to the root.
long double upper_tail_inverse(long double q) {
  const long double inv_sqrt2 = 0.70710678118654752440084436210484903928L;
  const long double inv_sqrt2pi = 0.39894228040143267793994605993438186848L;
  long double z = 0.0L;
  for (int it = 0; it < 200; ++it) {
    long double tail = 0.5L * erfcl(z * inv_sqrt2);
    long double dens = inv_sqrt2pi * expl(-0.5L * z * z);
    long double step = (tail - q) / dens;
    long double next = z + step;
    if (next == z) break;
    z = next;
  }
  return z;
}

void nf4_values(float out[16]) {
  const long double delta = 929.0L / 960.0L;
  const long double zmax = upper_tail_inverse(1.0L - delta);
  for (int j = 1; j <= 7; ++j) {
    long double p = 0.5L + (delta - 0.5L) * (long double)j / 7.0L;
    out[7 - j] = (float)(-upper_tail_inverse(1.0L - p) / zmax);
  }
  out[7] = 0.0f;
  for (int j = 1; j <= 8; ++j) {
    long double p = 0.5L + (delta - 0.5L) * (long double)j / 8.0L;
    out[7 + j] = (float)(upper_tail_inverse(1.0L - p) / zmax);
  }
  out[0] = -1.0f;
  out[15] = 1.0f;
}

void fp4_values(float out[16]) {
  static const long double kE2M1[8] = {0.0L, 0.5L, 1.0L, 1.5L, 2.0L, 3.0L, 4.0L, 6.0L};
  for (int nib = 0; nib < 16; ++nib) {
    long double v = kE2M1[nib & 7] / 6.0L;
    out[nib] = (float)((nib & 8) ? -v : v);
  }
}

// Round-down fp32 of a double.
float round_down_f32(double v) {
  float f = (float)v;
  if ((double)f > v) f = nextafterf(f, -INFINITY);
  return f;
}

void build(int quant_type, CodeTables &t) {
  if (quant_type == kQuantNF4)
    nf4_values(t.value);
  else
    fp4_values(t.value);

  // Candidate codes sorted by value; FP4 nibble 8 (-0) is never emitted.
  std::vector<int> codes;
  for (int c = 0; c < 16; ++c)
    if (!(quant_type == kQuantFP4 && c == 8)) codes.push_back(c);
  std::stable_sort(codes.begin(), codes.end(),
                   [&](int a, int b) { return t.value[a] < t.value[b]; });

  // Decision thresholds: code rank r is chosen for s with T[r-1] < s <= T[r],
  // T = the largest fp32 not above the exact midpoint of neighbouring values
  // (the sum of two fp32 values is exact in fp64). This is the nearest value,
  // with an exact tie going to the smaller one.
  const int nc = (int)codes.size();
  std::vector<float> thr(nc - 1);
  for (int r = 0; r + 1 < nc; ++r)
    thr[r] = round_down_f32(0.5 * ((double)t.value[codes[r]] + (double)t.value[codes[r + 1]]));

  // Cell lookup. The kernel computes u = RN(128 s + 128) exactly with one fma
  // and reads cell i = floor(u / 8); every s of cell i lies in
  // [(8i - 128.5)/128, (8i - 120.5)/128], width 1/16. The smallest gap between
  // thresholds (> 0.079) exceeds the cell width, so at most one threshold
  // falls inside a cell.
  for (int i = 0; i < kCells; ++i) {
    double lo = (8 * i - 128.5) / 128.0, hi = (8 * i - 120.5) / 128.0;
    int below = 0, inside = 0;
    float cut = 4.0f;  // above every s: never crossed
    for (int r = 0; r + 1 < nc; ++r) {
      if ((double)thr[r] < lo)
        ++below;
      else if ((double)thr[r] < hi) {
        ++inside;
        cut = thr[r];
      }
    }
    if (inside > 1) abort();  // impossible for these tables (gap > 1/16)
    const uint32_t cb = (uint32_t)codes[below];
    const uint32_t ca = (uint32_t)codes[std::min(below + inside, nc - 1)];
    t.cell_thr[i] = cut;
    t.cell_codes[i] = cb | (ca << 8) | (cb << 20) | (ca << 28);
  }
}

}  // namespace

const CodeTables &code_tables(int quant_type) {
  static CodeTables tables[2];
  static std::once_flag once;
  std::call_once(once, [] {
    build(kQuantNF4, tables[0]);
    build(kQuantFP4, tables[1]);
  });
  return tables[quant_type == kQuantFP4 ? 1 : 0];
}

}  // namespace nf4
