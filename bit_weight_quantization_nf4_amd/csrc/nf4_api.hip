// nf4_api.hip -- the extern "C" boundary of libnf4 (declared in include/nf4.h):
// argument validation, device checks and dispatch to the kernel launchers.
// Every check runs before the first launch, so a rejected call writes nothing.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "../../include/nf4.h"
#include "nf4_internal.h"

using namespace nf4;

namespace {

bool is_pow2_in(int64_t v, int64_t lo, int64_t hi) {
  return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int32_t d) {
  return d == NF4_DTYPE_BF16 || d == NF4_DTYPE_FP32 || d == NF4_DTYPE_FP16;
}

int64_t dtype_bytes(int32_t d) { return d == NF4_DTYPE_FP32 ? 4 : 2; }

// Per-device result of the architecture check: 0 unknown, 1 ok, 2 not gfx950.
std::atomic<int> g_arch_state[64];

nf4_status check_device() {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return NF4_ERR_DEVICE;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NF4_ERR_DEVICE;
  if (dev < 0 || dev >= 64) return NF4_ERR_DEVICE;
  int st = g_arch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NF4_ERR_DEVICE;
    st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? NF4_OK : NF4_ERR_UNSUPPORTED;
}

nf4_status from_hip(hipError_t e) {
  if (e == hipSuccess) return NF4_OK;
  return e == hipErrorNotSupported ? NF4_ERR_UNSUPPORTED : NF4_ERR_DEVICE;
}

std::atomic<int> g_cu_count[64];

// Validates a quantized-tensor descriptor; fills the kernels' scale source
// with only the arrays its double-quant mode reads (a caller may leave stale
// pointers in the others).
nf4_status check_qweight(const nf4_qweight *w, ScaleArgs *sc) {
  if (w == nullptr) return NF4_ERR_INVALID_ARGUMENT;
  if (w->n < 0) return NF4_ERR_INVALID_ARGUMENT;
  if (w->quant_type != NF4_QUANT_NF4 && w->quant_type != NF4_QUANT_FP4)
    return NF4_ERR_INVALID_ARGUMENT;
  if (!is_pow2_in(w->blocksize, 32, 4096)) return NF4_ERR_INVALID_ARGUMENT;
  const int dq = w->double_quant;
  if (dq != NF4_DQ_NONE && dq != NF4_DQ_SYMMETRIC && dq != NF4_DQ_CENTRED)
    return NF4_ERR_INVALID_ARGUMENT;
  if (w->n > 0 && w->packed == nullptr) return NF4_ERR_INVALID_ARGUMENT;
  if (dq != NF4_DQ_NONE) {
    if (!is_pow2_in(w->blocksize2, 64, 4096)) return NF4_ERR_INVALID_ARGUMENT;
    if (w->n > 0 && (w->absmax_q == nullptr || w->absmax_scale == nullptr))
      return NF4_ERR_INVALID_ARGUMENT;
    if (dq == NF4_DQ_CENTRED && w->n > 0 && w->absmax_offset == nullptr)
      return NF4_ERR_INVALID_ARGUMENT;
    if (!aligned16(w->absmax_q) || !aligned16(w->absmax_scale)) return NF4_ERR_MISALIGNED;
    if (dq == NF4_DQ_CENTRED && !aligned16(w->absmax_offset)) return NF4_ERR_MISALIGNED;
  } else {
    if (w->n > 0 && w->absmax == nullptr) return NF4_ERR_INVALID_ARGUMENT;
    if (!aligned16(w->absmax)) return NF4_ERR_MISALIGNED;
  }
  if (!aligned16(w->packed)) return NF4_ERR_MISALIGNED;
  sc->absmax = dq ? nullptr : w->absmax;
  sc->absmax_q = dq ? w->absmax_q : nullptr;
  sc->absmax_scale = dq ? w->absmax_scale : nullptr;
  sc->absmax_offset = dq == NF4_DQ_CENTRED ? w->absmax_offset : nullptr;
  sc->double_quant = dq;
  sc->log2_bs2 = dq ? __builtin_ctz((unsigned)w->blocksize2) : 0;
  return NF4_OK;
}

// The rules of one product: shapes, dtypes, strides (elements), alignment.
nf4_status check_product(const void *x, int64_t ldx, int32_t M, const nf4_qweight *w, int32_t N,
                         int32_t K, int32_t compute_dtype, int32_t out_dtype, const void *y,
                         int64_t ldy, const void *bias, ScaleArgs *sc) {
  nf4_status st = check_qweight(w, sc);
  if (st != NF4_OK) return st;
  if (M < 0 || N < 0 || K <= 0) return NF4_ERR_INVALID_ARGUMENT;
  if ((int64_t)N * (int64_t)K != w->n) return NF4_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(out_dtype) || !valid_dtype(compute_dtype)) return NF4_ERR_INVALID_ARGUMENT;
  if (ldx < K || ldy < N) return NF4_ERR_INVALID_ARGUMENT;
  if (K % w->blocksize != 0) return NF4_ERR_UNSUPPORTED;
  if (M > 0 && N > 0 && (x == nullptr || y == nullptr)) return NF4_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(y)) return NF4_ERR_MISALIGNED;
  const int64_t xe = dtype_bytes(compute_dtype), ye = dtype_bytes(out_dtype);
  // activation rows after the first must start 16-byte aligned as well (they
  // are read in 16-byte pieces); outputs are written element by element
  if (M > 1 && (ldx * xe) % 16 != 0) return NF4_ERR_MISALIGNED;
  if ((reinterpret_cast<uintptr_t>(bias) & (uintptr_t)(xe - 1)) != 0) return NF4_ERR_MISALIGNED;
  // the kernels address x and y of one call with 31-bit byte offsets
  if (M > 0 && ((int64_t)(M - 1) * ldx + K) * xe >= ((int64_t)1 << 31)) return NF4_ERR_UNSUPPORTED;
  if (M > 0 && ((int64_t)(M - 1) * ldy + N) * ye >= ((int64_t)1 << 31)) return NF4_ERR_UNSUPPORTED;
  return NF4_OK;
}

}  // namespace

int nf4::device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

extern "C" {

int32_t nf4_abi_version(void) { return NF4_ABI_VERSION; }

const char *nf4_status_string(int32_t status) {
  switch (status) {
    case NF4_OK:
      return "NF4_OK";
    case NF4_ERR_INVALID_ARGUMENT:
      return "NF4_ERR_INVALID_ARGUMENT: null pointer, negative size, unknown enum or shape mismatch";
    case NF4_ERR_UNSUPPORTED:
      return "NF4_ERR_UNSUPPORTED: request this library does not implement, or device is not gfx950";
    case NF4_ERR_MISALIGNED:
      return "NF4_ERR_MISALIGNED: a device pointer or row stride is not 16-byte aligned";
    case NF4_ERR_DEVICE:
      return "NF4_ERR_DEVICE: no HIP device, or a HIP call or kernel launch failed";
    case NF4_ERR_SCRATCH:
      return "NF4_ERR_SCRATCH: the product needs more workspace than the static scratch of "
             "nf4_linear_noalloc holds (NF4_NOALLOC_SCRATCH_BYTES)";
    default:
      return "unknown nf4 status";
  }
}

int64_t nf4_packed_bytes(int64_t n) { return n < 0 ? -1 : (n + 1) / 2; }

int64_t nf4_num_blocks(int64_t n, int32_t blocksize) {
  if (n < 0 || blocksize <= 0) return -1;
  return (n + blocksize - 1) / blocksize;
}

nf4_status nf4_codebook(int32_t quant_type, float values[16]) {
  if (values == nullptr) return NF4_ERR_INVALID_ARGUMENT;
  if (quant_type != NF4_QUANT_NF4 && quant_type != NF4_QUANT_FP4) return NF4_ERR_INVALID_ARGUMENT;
  const CodeTables &t = code_tables(quant_type);
  memcpy(values, t.value, sizeof t.value);
  return NF4_OK;
}

nf4_status nf4_device_check(void) { return check_device(); }

}  // extern "C"

namespace {

// The per-tensor output rules of the quantize calls (no device work).
nf4_status check_quant_outputs(int64_t n, int32_t blocksize, int32_t quant_type,
                               int32_t double_quant, const uint8_t *packed, const float *absmax,
                               const int8_t *absmax_q, const float *absmax_scale,
                               const float *absmax_offset) {
  if (n < 0) return NF4_ERR_INVALID_ARGUMENT;
  if (quant_type != NF4_QUANT_NF4 && quant_type != NF4_QUANT_FP4) return NF4_ERR_INVALID_ARGUMENT;
  if (!is_pow2_in(blocksize, 32, 4096)) return NF4_ERR_INVALID_ARGUMENT;
  if (double_quant != NF4_DQ_NONE && double_quant != NF4_DQ_SYMMETRIC &&
      double_quant != NF4_DQ_CENTRED)
    return NF4_ERR_INVALID_ARGUMENT;
  if (n > 0 && (packed == nullptr || absmax == nullptr)) return NF4_ERR_INVALID_ARGUMENT;
  if (double_quant && n > 0 && (absmax_q == nullptr || absmax_scale == nullptr))
    return NF4_ERR_INVALID_ARGUMENT;
  if (double_quant == NF4_DQ_CENTRED && n > 0 && absmax_offset == nullptr)
    return NF4_ERR_INVALID_ARGUMENT;
  if (!aligned16(packed) || !aligned16(absmax)) return NF4_ERR_MISALIGNED;
  if (double_quant && (!aligned16(absmax_q) || !aligned16(absmax_scale))) return NF4_ERR_MISALIGNED;
  if (double_quant == NF4_DQ_CENTRED && !aligned16(absmax_offset)) return NF4_ERR_MISALIGNED;
  return NF4_OK;
}

// The second level after a quantize launch (blocksize2 = 256).
nf4_status second_level(const QuantTensorDesc &d, int32_t blocksize, int32_t double_quant,
                        float *absmax_offset, hipStream_t s) {
  const int64_t nb = (d.n + blocksize - 1) / blocksize;
  if (double_quant == NF4_DQ_SYMMETRIC)
    return from_hip(launch_double_quant(d.absmax, nb, 256, d.absmax_q, d.absmax_scale, s));
  if (double_quant == NF4_DQ_CENTRED)
    return from_hip(launch_double_quant_centred(d.absmax, nb, 256, d.absmax_q, d.absmax_scale,
                                                absmax_offset, s));
  return NF4_OK;
}

}  // namespace

extern "C" {

nf4_status nf4_quantize(const void *w_bf16, int64_t n, int32_t blocksize, int32_t quant_type,
                        int32_t double_quant, uint8_t *packed, float *absmax, int8_t *absmax_q,
                        float *absmax_scale, void *stream) {
  return nf4_quantize_grouped(1, &w_bf16, &n, blocksize, quant_type, double_quant, &packed,
                              &absmax, &absmax_q, &absmax_scale, stream);
}

nf4_status nf4_quantize_grouped(int32_t count, const void *const *w_bf16, const int64_t *n,
                                int32_t blocksize, int32_t quant_type, int32_t double_quant,
                                uint8_t *const *packed, float *const *absmax,
                                int8_t *const *absmax_q, float *const *absmax_scale,
                                void *stream) {
  if (count < 0 || count > NF4_QUANT_MAX_GROUP) return NF4_ERR_INVALID_ARGUMENT;
  if (count == 0) return NF4_OK;
  if (w_bf16 == nullptr || n == nullptr || packed == nullptr || absmax == nullptr)
    return NF4_ERR_INVALID_ARGUMENT;
  // these calls take the symmetric second level only (no offset array)
  if (double_quant != NF4_DQ_NONE && double_quant != NF4_DQ_SYMMETRIC)
    return NF4_ERR_INVALID_ARGUMENT;
  if (double_quant == NF4_DQ_SYMMETRIC && (absmax_q == nullptr || absmax_scale == nullptr))
    return NF4_ERR_INVALID_ARGUMENT;
  QuantTensorDesc ds[NF4_QUANT_MAX_GROUP];
  bool any = false;
  for (int i = 0; i < count; ++i) {
    int8_t *q = double_quant ? absmax_q[i] : nullptr;
    float *s2 = double_quant ? absmax_scale[i] : nullptr;
    nf4_status st = check_quant_outputs(n[i], blocksize, quant_type, double_quant, packed[i],
                                        absmax[i], q, s2, nullptr);
    if (st != NF4_OK) return st;
    if (n[i] > 0 && w_bf16[i] == nullptr) return NF4_ERR_INVALID_ARGUMENT;
    if (!aligned16(w_bf16[i])) return NF4_ERR_MISALIGNED;
    ds[i] = QuantTensorDesc{static_cast<const uint16_t *>(w_bf16[i]), n[i], packed[i], absmax[i],
                            q, s2};
    any = any || n[i] > 0;
  }
  if (!any) return NF4_OK;
  nf4_status st = check_device();
  if (st != NF4_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool fused = double_quant && quantize_dq_fused(blocksize, 256);
  if (log_on())
    log_msg("quantize %d tensor(s) (first n=%lld) bs=%d: %s", count, (long long)n[0], blocksize,
            fused ? "quantize_dq_kernel (double quant in the same pass)"
                  : double_quant ? "quantize_kernel, then the second level" : "quantize_kernel");
  if (fused) return from_hip(launch_quantize_dq(count, ds, blocksize, quant_type, s));
  for (int i = 0; i < count && st == NF4_OK; ++i) {
    if (ds[i].n == 0) continue;
    st = from_hip(
        launch_quantize(ds[i].w, ds[i].n, blocksize, quant_type, ds[i].packed, ds[i].absmax, s));
    if (st == NF4_OK) st = second_level(ds[i], blocksize, double_quant, nullptr, s);
  }
  return st;
}

nf4_status nf4_quantize_ex(const void *w, int32_t w_dtype, int64_t rows, int64_t cols, int64_t ld,
                           int32_t blocksize, int32_t quant_type, int32_t double_quant,
                           uint8_t *packed, float *absmax, int8_t *absmax_q, float *absmax_scale,
                           float *absmax_offset, void *stream) {
  if (!valid_dtype(w_dtype)) return NF4_ERR_INVALID_ARGUMENT;
  if (rows < 0 || cols < 0 || ld < cols) return NF4_ERR_INVALID_ARGUMENT;
  if (cols > 0 && rows > INT64_MAX / cols) return NF4_ERR_INVALID_ARGUMENT;
  const int64_t n = rows * cols;
  nf4_status st = check_quant_outputs(n, blocksize, quant_type, double_quant, packed, absmax,
                                      absmax_q, absmax_scale, absmax_offset);
  if (st != NF4_OK) return st;
  if (n > 0 && w == nullptr) return NF4_ERR_INVALID_ARGUMENT;
  if (!aligned16(w)) return NF4_ERR_MISALIGNED;
  const bool strided = rows > 1 && ld != cols;
  if (strided) {
    if (cols % 8 != 0) return NF4_ERR_UNSUPPORTED;
    if ((ld * dtype_bytes(w_dtype)) % 16 != 0) return NF4_ERR_MISALIGNED;
  }
  if (n == 0) return NF4_OK;
  st = check_device();
  if (st != NF4_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  QuantTensorDesc d{static_cast<const uint16_t *>(w), n, packed, absmax, absmax_q, absmax_scale};
  if (log_on())
    log_msg("quantize rows=%lld cols=%lld ld=%lld dtype=%d bs=%d double_quant=%d: %s",
            (long long)rows, (long long)cols, (long long)ld, w_dtype, blocksize, double_quant,
            w_dtype == NF4_DTYPE_BF16 && !strided ? "bf16 kernels" : "quantize_generic_kernel");
  if (w_dtype == NF4_DTYPE_BF16 && !strided) {
    // the bf16 kernels (one pass with the symmetric second level at 64/128/256)
    if (double_quant == NF4_DQ_SYMMETRIC && quantize_dq_fused(blocksize, 256))
      return from_hip(launch_quantize_dq(1, &d, blocksize, quant_type, s));
    st = from_hip(launch_quantize(d.w, n, blocksize, quant_type, packed, absmax, s));
  } else {
    st = from_hip(launch_quantize_generic(w, w_dtype, rows, cols, rows > 1 ? ld : cols,
                                          blocksize, quant_type, packed, absmax, s));
  }
  if (st != NF4_OK) return st;
  return second_level(d, blocksize, double_quant, absmax_offset, s);
}

nf4_status nf4_double_quant(const float *absmax, int64_t nb, int32_t blocksize2, int8_t *absmax_q,
                            float *absmax_scale, void *stream) {
  return nf4_double_quant_ex(absmax, nb, blocksize2, NF4_DQ_SYMMETRIC, absmax_q, absmax_scale,
                             nullptr, stream);
}

nf4_status nf4_double_quant_ex(const float *absmax, int64_t nb, int32_t blocksize2, int32_t mode,
                               int8_t *absmax_q, float *absmax_scale, float *absmax_offset,
                               void *stream) {
  if (nb < 0) return NF4_ERR_INVALID_ARGUMENT;
  if (mode != NF4_DQ_SYMMETRIC && mode != NF4_DQ_CENTRED) return NF4_ERR_INVALID_ARGUMENT;
  if (!is_pow2_in(blocksize2, 64, 4096)) return NF4_ERR_INVALID_ARGUMENT;
  if (nb > 0 && (absmax == nullptr || absmax_q == nullptr || absmax_scale == nullptr))
    return NF4_ERR_INVALID_ARGUMENT;
  if (mode == NF4_DQ_CENTRED && nb > 0 && absmax_offset == nullptr)
    return NF4_ERR_INVALID_ARGUMENT;
  if (!aligned16(absmax) || !aligned16(absmax_q) || !aligned16(absmax_scale))
    return NF4_ERR_MISALIGNED;
  if (mode == NF4_DQ_CENTRED && !aligned16(absmax_offset)) return NF4_ERR_MISALIGNED;
  if (nb == 0) return NF4_OK;
  nf4_status st = check_device();
  if (st != NF4_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (mode == NF4_DQ_CENTRED)
    return from_hip(launch_double_quant_centred(absmax, nb, blocksize2, absmax_q, absmax_scale,
                                                absmax_offset, s));
  return from_hip(launch_double_quant(absmax, nb, blocksize2, absmax_q, absmax_scale, s));
}

nf4_status nf4_dequantize(const nf4_qweight *w, int32_t out_dtype, void *out, void *stream) {
  return nf4_dequantize_grouped(1, w, out_dtype, &out, stream);
}

nf4_status nf4_dequantize_grouped(int32_t count, const nf4_qweight *w, int32_t out_dtype,
                                  void *const *out, void *stream) {
  if (count < 0 || count > NF4_QUANT_MAX_GROUP) return NF4_ERR_INVALID_ARGUMENT;
  if (count == 0) return NF4_OK;
  if (w == nullptr || out == nullptr) return NF4_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(out_dtype)) return NF4_ERR_INVALID_ARGUMENT;
  DequantDesc ds[NF4_QUANT_MAX_GROUP];
  bool any = false;
  for (int i = 0; i < count; ++i) {
    ScaleArgs sc;
    nf4_status st = check_qweight(&w[i], &sc);
    if (st != NF4_OK) return st;
    if (w[i].n > 0 && out[i] == nullptr) return NF4_ERR_INVALID_ARGUMENT;
    if (!aligned16(out[i])) return NF4_ERR_MISALIGNED;
    if (w[i].quant_type != w[0].quant_type || w[i].double_quant != w[0].double_quant)
      return NF4_ERR_UNSUPPORTED;
    ds[i] = DequantDesc{w[i].packed, w[i].n, w[i].blocksize, sc, out[i]};
    any = any || w[i].n > 0;
  }
  if (!any) return NF4_OK;
  nf4_status st = check_device();
  if (st != NF4_OK) return st;
  if (log_on())
    log_msg("dequantize %d tensor(s) (first n=%lld) out_dtype=%d: dequantize_kernel", count,
            (long long)w[0].n, out_dtype);
  return from_hip(launch_dequantize(count, ds, w[0].quant_type, w[0].double_quant, out_dtype,
                                    reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// NF4_FORCE_KERNEL=mfma in the environment sends M = 1 products to the
// matrix-core decode kernel instead of the single-row kernel (for A/B
// measurement); read once per process.
bool force_mfma_decode() {
  static const bool force = [] {
    const char *v = getenv("NF4_FORCE_KERNEL");
    return v != nullptr && strcmp(v, "mfma") == 0;
  }();
  return force;
}

// The single-row kernel takes M = 1 products with a bf16 compute dtype, a bf16
// or fp32 output and at most the symmetric second level, up to its longest K
// (which depends on the blocksize).
bool single_row_path(int32_t M, int32_t K, int32_t blocksize, int32_t compute_dtype,
                     int32_t out_dtype, int dq) {
  return M == 1 && compute_dtype == NF4_DTYPE_BF16 && out_dtype != NF4_DTYPE_FP16 &&
         dq != NF4_DQ_CENTRED && K <= gemv1_max_k(blocksize) && !force_mfma_decode();
}

// The decode products of a grouped call (each with an optional bias; bias ==
// nullptr: none), on the kernels their own (M, K, dtypes, mode) select, so a
// product's result never depends on what it is grouped with.
nf4_status gemv_grouped_impl(int32_t count, const void *const *x, const int64_t *ldx, int32_t M,
                             const nf4_qweight *w, const int32_t *N, const int32_t *K,
                             const void *const *bias, int32_t compute_dtype, int32_t out_dtype,
                             void *const *y, const int64_t *ldy, void *workspace,
                             int64_t workspace_bytes, void *stream) {
  if (count < 0 || count > NF4_GEMV_MAX_GROUP) return NF4_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < 0 || (workspace_bytes > 0 && workspace == nullptr))
    return NF4_ERR_INVALID_ARGUMENT;
  if (!aligned16(workspace)) return NF4_ERR_MISALIGNED;
  if (count == 0) return NF4_OK;
  if (x == nullptr || w == nullptr || N == nullptr || K == nullptr || y == nullptr)
    return NF4_ERR_INVALID_ARGUMENT;
  GemvDesc descs[NF4_GEMV_MAX_GROUP];
  for (int i = 0; i < count; ++i) {
    ScaleArgs sc;
    const int64_t lx = ldx ? ldx[i] : K[i], ly = ldy ? ldy[i] : N[i];
    const void *b = bias ? bias[i] : nullptr;
    nf4_status st = check_product(x[i], lx, M, &w[i], N[i], K[i], compute_dtype, out_dtype, y[i],
                                  ly, b, &sc);
    if (st != NF4_OK) return st;
    if (w[i].quant_type != w[0].quant_type || w[i].double_quant != w[0].double_quant)
      return NF4_ERR_UNSUPPORTED;
    descs[i] = GemvDesc{x[i], w[i].packed, y[i], sc, N[i], K[i], w[i].blocksize, b, lx, ly};
  }
  if (M > NF4_GEMV_MAX_M) return NF4_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < count; ++i)
    if (K[i] > (1 << 24)) return NF4_ERR_UNSUPPORTED;  // 31-bit offsets within a work item
  if (M == 0) return NF4_OK;
  nf4_status st = check_device();
  if (st != NF4_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int dq = w[0].double_quant, qt = w[0].quant_type;
  if (compute_dtype == NF4_DTYPE_FP32) {
    for (int i = 0; i < count && st == NF4_OK; ++i) {
      if (log_on() && descs[i].N > 0)
        log_msg("product M=%d N=%d K=%d: matmul_f32_kernel (fp32 compute)", M, descs[i].N, K[i]);
      if (descs[i].N > 0) st = from_hip(launch_matmul_f32(descs[i], M, qt, out_dtype, s));
    }
    return st;
  }
  GemvDesc one[NF4_GEMV_MAX_GROUP];
  int n_one = 0;
  bool done[NF4_GEMV_MAX_GROUP] = {};
  for (int i = 0; i < count; ++i)
    if (single_row_path(M, K[i], w[i].blocksize, compute_dtype, out_dtype, dq)) {
      one[n_one++] = descs[i];
      done[i] = true;
    }
  if (n_one > 0) {
    if (log_on())
      log_msg("decode M=1: gemv1_kernel, %d product(s) in one launch (first N=%d K=%d)", n_one,
              one[0].N, one[0].K);
    st = from_hip(launch_gemv1_grouped(n_one, one, qt, dq != NF4_DQ_NONE,
                                       out_dtype == NF4_DTYPE_BF16, s));
    if (st != NF4_OK) return st;
  }
  // the rest on the matrix-core kernels, one launch per distinct (K,
  // blocksize); launches on one stream run in order, so each may use the
  // whole workspace
  for (int i = 0; i < count && st == NF4_OK; ++i) {
    if (done[i]) continue;
    GemvDesc same[NF4_GEMV_MAX_GROUP];
    int ns = 0;
    for (int j = i; j < count; ++j)
      if (!done[j] && K[j] == K[i] && w[j].blocksize == w[i].blocksize) {
        same[ns++] = descs[j];
        done[j] = true;
      }
    st = from_hip(launch_gemv_mt(ns, same, M, K[i], qt, dq, compute_dtype, out_dtype, workspace,
                                 (size_t)workspace_bytes, s));
  }
  return st;
}

// Prefill products of at least NF4_PREFILL_DEQUANT_MIN_M rows dequantize the
// weight once into the workspace and run the GEMM on it, instead of
// dequantizing each weight tile again for every 256-row tile of x inside the
// GEMM (measured on the 14336 x 4096 weight: 2048 rows 230-236 against
// 260-274 us; 1024 and 512 rows about even).
constexpr int32_t kPrefillDequantMinM = NF4_PREFILL_DEQUANT_MIN_M;

// Bytes of the dequantized weight a prefill product takes, 0 when it takes the
// fused GEMM.
int64_t prefill_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t compute_dtype) {
  if (M < kPrefillDequantMinM || N <= 0 || K <= 0) return 0;
  if (compute_dtype != NF4_DTYPE_BF16 && compute_dtype != NF4_DTYPE_FP16) return 0;
  return ((2 * (int64_t)N * K) + 255) / 256 * 256;
}

// Workspace bytes a product takes: the K split of the matrix-core decode
// kernel, or the dequantized weight of a prefill product; 0 when its dispatch
// uses none.
int64_t product_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t blocksize,
                                int32_t compute_dtype, int32_t out_dtype, int dq) {
  if (M > NF4_GEMV_MAX_M) return prefill_workspace_bytes(M, N, K, compute_dtype);
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  if (compute_dtype == NF4_DTYPE_FP32) return 0;
  if (single_row_path(M, K, blocksize, compute_dtype, out_dtype, dq)) return 0;
  return (int64_t)gemv_split_bytes(M, N, K);
}

nf4_status gemm_impl(const void *x, int64_t ldx, int32_t M, const nf4_qweight *w, int32_t N,
                     int32_t K, const void *bias, int32_t compute_dtype, int32_t out_dtype,
                     void *y, int64_t ldy, void *stream, void *workspace = nullptr,
                     int64_t workspace_bytes = 0) {
  ScaleArgs sc;
  nf4_status st =
      check_product(x, ldx, M, w, N, K, compute_dtype, out_dtype, y, ldy, bias, &sc);
  if (st != NF4_OK) return st;
  // a tile's offsets into x, the codes and y are 32-bit
  if (K > (1 << 22) || N > (1 << 21)) return NF4_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return NF4_OK;
  st = check_device();
  if (st != NF4_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (compute_dtype == NF4_DTYPE_FP32) {
    const GemvDesc d{x, w->packed, y, sc, N, K, w->blocksize, bias, ldx, ldy};
    if (log_on()) log_msg("product M=%d N=%d K=%d: matmul_f32_kernel (fp32 compute)", M, N, K);
    return from_hip(launch_matmul_f32(d, M, w->quant_type, out_dtype, s));
  }
  const int64_t need = prefill_workspace_bytes(M, N, K, compute_dtype);
  if (need > 0 && workspace_bytes >= need) {
    // the weight once in the compute dtype (the dequantize kernel's values,
    // the ones the fused GEMM forms tile by tile), then the GEMM on it
    DequantDesc d{w->packed, (int64_t)N * K, w->blocksize, sc, workspace};
    if (log_on())
      log_msg("prefill M=%d N=%d K=%d bs=%d: dequantize once into the workspace (%lld bytes), "
              "then gemm_w16_kernel", M, N, K, w->blocksize, (long long)need);
    hipError_t e = launch_dequantize(1, &d, w->quant_type, sc.double_quant, compute_dtype, s);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(launch_gemm_w16(x, ldx, M, workspace, K, N, K, compute_dtype, out_dtype, y,
                                    ldy, bias, s));
  }
  if (log_on())
    log_msg("prefill M=%d N=%d K=%d bs=%d: gemm_kernel (dequantization fused)%s", M, N, K,
            w->blocksize, need > 0 ? "; workspace below the 2 N K bytes it would use" : "");
  return from_hip(launch_gemm(x, ldx, M, w->packed, N, K, w->blocksize, w->quant_type, sc,
                              compute_dtype, out_dtype, y, ldy, bias, s));
}

nf4_status linear_impl(const void *x, int64_t ldx, int32_t M, const nf4_qweight *w, int32_t N,
                       int32_t K, const void *bias, int32_t compute_dtype, int32_t out_dtype,
                       void *y, int64_t ldy, void *workspace, int64_t workspace_bytes,
                       void *stream) {
  // decode shapes take the decode kernels, larger batches the prefill GEMM
  if (M >= 0 && M <= NF4_GEMV_MAX_M)
    return gemv_grouped_impl(1, &x, &ldx, M, w, &N, &K, &bias, compute_dtype, out_dtype, &y, &ldy,
                             workspace, workspace_bytes, stream);
  if (workspace_bytes < 0 || (workspace_bytes > 0 && workspace == nullptr))
    return NF4_ERR_INVALID_ARGUMENT;
  if (!aligned16(workspace)) return NF4_ERR_MISALIGNED;
  return gemm_impl(x, ldx, M, w, N, K, bias, compute_dtype, out_dtype, y, ldy, stream, workspace,
                   workspace_bytes);
}

}  // namespace

namespace nf4 {

bool log_on() {
  static const bool on = [] {
    const char *v = getenv("NF4_LOG");
    return v != nullptr && *v != '\0' && strcmp(v, "0") != 0;
  }();
  return on;
}

void log_msg(const char *fmt, ...) {
  char line[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(line, sizeof line, fmt, ap);
  va_end(ap);
  fprintf(stderr, "[nf4] %s\n", line);
}

nf4_status linear_with_workspace(const void *x, int64_t ldx, int32_t M, const nf4_qweight *w,
                                 int32_t N, int32_t K, const void *bias, int32_t compute_dtype,
                                 int32_t out_dtype, void *y, int64_t ldy, void *workspace,
                                 int64_t workspace_bytes, void *stream) {
  return linear_impl(x, ldx, M, w, N, K, bias, compute_dtype, out_dtype, y, ldy, workspace,
                     workspace_bytes, stream);
}

int64_t linear_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t blocksize,
                               int32_t compute_dtype, int32_t out_dtype, int32_t double_quant) {
  return product_workspace_bytes(M, N, K, blocksize, compute_dtype, out_dtype, double_quant);
}

}  // namespace nf4

extern "C" {

nf4_status nf4_gemv(const void *x, int32_t M, const nf4_qweight *w, int32_t N, int32_t K,
                    int32_t compute_dtype, int32_t out_dtype, void *y, void *stream) {
  return gemv_grouped_impl(1, &x, nullptr, M, w, &N, &K, nullptr, compute_dtype, out_dtype, &y,
                           nullptr, nullptr, 0, stream);
}

nf4_status nf4_gemv_grouped(int32_t count, const void *const *x, int32_t M,
                            const nf4_qweight *w, const int32_t *N, const int32_t *K,
                            int32_t compute_dtype, int32_t out_dtype, void *const *y,
                            void *stream) {
  return gemv_grouped_impl(count, x, nullptr, M, w, N, K, nullptr, compute_dtype, out_dtype, y,
                           nullptr, nullptr, 0, stream);
}

nf4_status nf4_gemv_grouped_ws(int32_t count, const void *const *x, int32_t M,
                               const nf4_qweight *w, const int32_t *N, const int32_t *K,
                               int32_t compute_dtype, int32_t out_dtype, void *const *y,
                               void *workspace, int64_t workspace_bytes, void *stream) {
  return gemv_grouped_impl(count, x, nullptr, M, w, N, K, nullptr, compute_dtype, out_dtype, y,
                           nullptr, workspace, workspace_bytes, stream);
}

int64_t nf4_linear_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t blocksize,
                                   int32_t compute_dtype, int32_t out_dtype,
                                   int32_t double_quant) {
  return product_workspace_bytes(M, N, K, blocksize, compute_dtype, out_dtype, double_quant);
}

nf4_status nf4_gemm(const void *x, int32_t M, const nf4_qweight *w, int32_t N, int32_t K,
                    int32_t compute_dtype, int32_t out_dtype, void *y, void *stream) {
  return gemm_impl(x, K, M, w, N, K, nullptr, compute_dtype, out_dtype, y, N, stream);
}

nf4_status nf4_linear(const void *x, int32_t M, const nf4_qweight *w, int32_t N, int32_t K,
                      const void *bias, int32_t compute_dtype, int32_t out_dtype, void *y,
                      void *stream) {
  return linear_impl(x, K, M, w, N, K, bias, compute_dtype, out_dtype, y, N, nullptr, 0, stream);
}

nf4_status nf4_linear_ex(const void *x, int64_t ldx, int32_t M, const nf4_qweight *w, int32_t N,
                         int32_t K, const void *bias, int32_t compute_dtype, int32_t out_dtype,
                         void *y, int64_t ldy, void *stream) {
  return linear_impl(x, ldx, M, w, N, K, bias, compute_dtype, out_dtype, y, ldy, nullptr, 0,
                     stream);
}

nf4_status nf4_linear_ws(const void *x, int64_t ldx, int32_t M, const nf4_qweight *w, int32_t N,
                         int32_t K, const void *bias, int32_t compute_dtype, int32_t out_dtype,
                         void *y, int64_t ldy, void *workspace, int64_t workspace_bytes,
                         void *stream) {
  return linear_impl(x, ldx, M, w, N, K, bias, compute_dtype, out_dtype, y, ldy, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"
