// nf4_api.hip -- the extern "C" boundary of libnf4 (declared in include/nf4.h):
// argument validation, device checks and dispatch to the kernel launchers.
// Every check runs before the first launch, so a rejected call writes nothing.
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

nf4_status from_hip(hipError_t e) { return e == hipSuccess ? NF4_OK : NF4_ERR_DEVICE; }

std::atomic<int> g_cu_count[64];

// Validates a quantized-tensor descriptor; fills the kernels' scale source.
nf4_status check_qweight(const nf4_qweight *w, ScaleArgs *sc) {
  if (w == nullptr) return NF4_ERR_INVALID_ARGUMENT;
  if (w->n < 0) return NF4_ERR_INVALID_ARGUMENT;
  if (w->quant_type != NF4_QUANT_NF4 && w->quant_type != NF4_QUANT_FP4)
    return NF4_ERR_INVALID_ARGUMENT;
  if (!is_pow2_in(w->blocksize, 32, 4096)) return NF4_ERR_INVALID_ARGUMENT;
  if (w->double_quant != 0 && w->double_quant != 1) return NF4_ERR_INVALID_ARGUMENT;
  if (w->n > 0 && w->packed == nullptr) return NF4_ERR_INVALID_ARGUMENT;
  if (w->double_quant) {
    if (!is_pow2_in(w->blocksize2, 64, 4096)) return NF4_ERR_INVALID_ARGUMENT;
    if (w->n > 0 && (w->absmax_q == nullptr || w->absmax_scale == nullptr))
      return NF4_ERR_INVALID_ARGUMENT;
    if (!aligned16(w->absmax_q) || !aligned16(w->absmax_scale)) return NF4_ERR_MISALIGNED;
  } else {
    if (w->n > 0 && w->absmax == nullptr) return NF4_ERR_INVALID_ARGUMENT;
    if (!aligned16(w->absmax)) return NF4_ERR_MISALIGNED;
  }
  if (!aligned16(w->packed)) return NF4_ERR_MISALIGNED;
  // only the scale arrays the flag selects reach the kernels: a caller may
  // leave stale pointers in the fields the mode does not read
  sc->absmax = w->double_quant ? nullptr : w->absmax;
  sc->absmax_q = w->double_quant ? w->absmax_q : nullptr;
  sc->absmax_scale = w->double_quant ? w->absmax_scale : nullptr;
  sc->double_quant = w->double_quant;
  sc->log2_bs2 = w->double_quant ? __builtin_ctz((unsigned)w->blocksize2) : 0;
  return NF4_OK;
}

nf4_status check_product(const void *x, int32_t M, const nf4_qweight *w, int32_t N, int32_t K,
                         int32_t compute_dtype, int32_t out_dtype, void *y, ScaleArgs *sc) {
  nf4_status st = check_qweight(w, sc);
  if (st != NF4_OK) return st;
  if (M < 0 || N < 0 || K <= 0) return NF4_ERR_INVALID_ARGUMENT;
  if ((int64_t)N * (int64_t)K != w->n) return NF4_ERR_INVALID_ARGUMENT;
  if (out_dtype != NF4_DTYPE_BF16 && out_dtype != NF4_DTYPE_FP32) return NF4_ERR_INVALID_ARGUMENT;
  if (compute_dtype != NF4_DTYPE_BF16 && compute_dtype != NF4_DTYPE_FP32)
    return NF4_ERR_INVALID_ARGUMENT;
  if (compute_dtype != NF4_DTYPE_BF16) return NF4_ERR_UNSUPPORTED;
  if (K % w->blocksize != 0) return NF4_ERR_UNSUPPORTED;
  if (M > 0 && N > 0 && (x == nullptr || y == nullptr)) return NF4_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(y)) return NF4_ERR_MISALIGNED;
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
      return "NF4_ERR_MISALIGNED: a device pointer is not 16-byte aligned";
    case NF4_ERR_DEVICE:
      return "NF4_ERR_DEVICE: no HIP device, or a HIP call or kernel launch failed";
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

namespace {

// The per-tensor rules of nf4_quantize (no device work).
nf4_status check_quantize(const void *w_bf16, int64_t n, int32_t blocksize, int32_t quant_type,
                          int32_t double_quant, const uint8_t *packed, const float *absmax,
                          const int8_t *absmax_q, const float *absmax_scale) {
  if (n < 0) return NF4_ERR_INVALID_ARGUMENT;
  if (quant_type != NF4_QUANT_NF4 && quant_type != NF4_QUANT_FP4) return NF4_ERR_INVALID_ARGUMENT;
  if (!is_pow2_in(blocksize, 32, 4096)) return NF4_ERR_INVALID_ARGUMENT;
  if (double_quant != 0 && double_quant != 1) return NF4_ERR_INVALID_ARGUMENT;
  if (n > 0 && (w_bf16 == nullptr || packed == nullptr || absmax == nullptr))
    return NF4_ERR_INVALID_ARGUMENT;
  if (double_quant && n > 0 && (absmax_q == nullptr || absmax_scale == nullptr))
    return NF4_ERR_INVALID_ARGUMENT;
  if (!aligned16(w_bf16) || !aligned16(packed) || !aligned16(absmax)) return NF4_ERR_MISALIGNED;
  if (double_quant && (!aligned16(absmax_q) || !aligned16(absmax_scale))) return NF4_ERR_MISALIGNED;
  return NF4_OK;
}

// One tensor through the launches that do not share a launch with others.
nf4_status quantize_one(const QuantTensorDesc &d, int32_t blocksize, int32_t quant_type,
                        int32_t double_quant, hipStream_t s) {
  if (d.n == 0) return NF4_OK;
  nf4_status st =
      from_hip(launch_quantize(d.w, d.n, blocksize, quant_type, d.packed, d.absmax, s));
  if (st != NF4_OK || !double_quant) return st;
  const int64_t nb = (d.n + blocksize - 1) / blocksize;
  return from_hip(launch_double_quant(d.absmax, nb, 256, d.absmax_q, d.absmax_scale, s));
}

}  // namespace

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
  if (double_quant == 1 && (absmax_q == nullptr || absmax_scale == nullptr))
    return NF4_ERR_INVALID_ARGUMENT;
  QuantTensorDesc ds[NF4_QUANT_MAX_GROUP];
  bool any = false;
  for (int i = 0; i < count; ++i) {
    int8_t *q = double_quant == 1 ? absmax_q[i] : nullptr;
    float *s2 = double_quant == 1 ? absmax_scale[i] : nullptr;
    nf4_status st = check_quantize(w_bf16[i], n[i], blocksize, quant_type, double_quant, packed[i],
                                   absmax[i], q, s2);
    if (st != NF4_OK) return st;
    ds[i] = QuantTensorDesc{static_cast<const uint16_t *>(w_bf16[i]), n[i], packed[i], absmax[i],
                            q, s2};
    any = any || n[i] > 0;
  }
  if (!any) return NF4_OK;
  nf4_status st = check_device();
  if (st != NF4_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (double_quant && quantize_dq_fused(blocksize, 256))
    return from_hip(launch_quantize_dq(count, ds, blocksize, quant_type, s));
  for (int i = 0; i < count && st == NF4_OK; ++i)
    st = quantize_one(ds[i], blocksize, quant_type, double_quant, s);
  return st;
}

nf4_status nf4_double_quant(const float *absmax, int64_t nb, int32_t blocksize2, int8_t *absmax_q,
                            float *absmax_scale, void *stream) {
  if (nb < 0) return NF4_ERR_INVALID_ARGUMENT;
  if (!is_pow2_in(blocksize2, 64, 4096)) return NF4_ERR_INVALID_ARGUMENT;
  if (nb > 0 && (absmax == nullptr || absmax_q == nullptr || absmax_scale == nullptr))
    return NF4_ERR_INVALID_ARGUMENT;
  if (!aligned16(absmax) || !aligned16(absmax_q) || !aligned16(absmax_scale))
    return NF4_ERR_MISALIGNED;
  if (nb == 0) return NF4_OK;
  nf4_status st = check_device();
  if (st != NF4_OK) return st;
  return from_hip(launch_double_quant(absmax, nb, blocksize2, absmax_q, absmax_scale,
                                      reinterpret_cast<hipStream_t>(stream)));
}

nf4_status nf4_dequantize(const nf4_qweight *w, int32_t out_dtype, void *out, void *stream) {
  return nf4_dequantize_grouped(1, w, out_dtype, &out, stream);
}

nf4_status nf4_dequantize_grouped(int32_t count, const nf4_qweight *w, int32_t out_dtype,
                                  void *const *out, void *stream) {
  if (count < 0 || count > NF4_QUANT_MAX_GROUP) return NF4_ERR_INVALID_ARGUMENT;
  if (count == 0) return NF4_OK;
  if (w == nullptr || out == nullptr) return NF4_ERR_INVALID_ARGUMENT;
  if (out_dtype != NF4_DTYPE_BF16 && out_dtype != NF4_DTYPE_FP32) return NF4_ERR_INVALID_ARGUMENT;
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
  return from_hip(launch_dequantize(count, ds, w[0].quant_type, w[0].double_quant != 0,
                                    out_dtype == NF4_DTYPE_BF16,
                                    reinterpret_cast<hipStream_t>(stream)));
}

nf4_status nf4_gemv(const void *x_bf16, int32_t M, const nf4_qweight *w, int32_t N, int32_t K,
                    int32_t compute_dtype, int32_t out_dtype, void *y, void *stream) {
  return nf4_gemv_grouped(1, &x_bf16, M, w, &N, &K, compute_dtype, out_dtype, &y, stream);
}

// the grouped decode products, each with an optional bias (bias == nullptr:
// none for any product)
static nf4_status gemv_grouped_impl(int32_t count, const void *const *x_bf16, int32_t M,
                                    const nf4_qweight *w, const int32_t *N, const int32_t *K,
                                    const void *const *bias, int32_t compute_dtype,
                                    int32_t out_dtype, void *const *y, void *stream) {
  if (count < 0 || count > NF4_GEMV_MAX_GROUP) return NF4_ERR_INVALID_ARGUMENT;
  if (count == 0) return NF4_OK;
  if (x_bf16 == nullptr || w == nullptr || N == nullptr || K == nullptr || y == nullptr)
    return NF4_ERR_INVALID_ARGUMENT;
  GemvDesc descs[NF4_GEMV_MAX_GROUP];
  for (int i = 0; i < count; ++i) {
    ScaleArgs sc;
    nf4_status st =
        check_product(x_bf16[i], M, &w[i], N[i], K[i], compute_dtype, out_dtype, y[i], &sc);
    if (st != NF4_OK) return st;
    if (w[i].quant_type != w[0].quant_type || w[i].double_quant != w[0].double_quant)
      return NF4_ERR_UNSUPPORTED;
    const uint16_t *b = bias ? static_cast<const uint16_t *>(bias[i]) : nullptr;
    if ((reinterpret_cast<uintptr_t>(b) & 1u) != 0) return NF4_ERR_MISALIGNED;
    descs[i] = GemvDesc{static_cast<const uint16_t *>(x_bf16[i]), w[i].packed, y[i], sc, N[i],
                        K[i], w[i].blocksize, b};
  }
  if (M > NF4_GEMV_MAX_M) return NF4_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < count; ++i)
    if (K[i] > (1 << 26)) return NF4_ERR_UNSUPPORTED;  // 31-bit activation offsets
  if (M == 0) return NF4_OK;
  nf4_status st = check_device();
  if (st != NF4_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool dq = w[0].double_quant != 0, bf16_out = out_dtype == NF4_DTYPE_BF16;
  if (M > 1)
    return from_hip(launch_gemv_grouped(count, descs, M, w[0].quant_type, dq, bf16_out, s));
  // M = 1: the single-row kernel takes the rows it can, the batched kernel the
  // longer ones (one launch each), so every product is computed exactly as
  // it would be on its own
  GemvDesc one[NF4_GEMV_MAX_GROUP], many[NF4_GEMV_MAX_GROUP];
  int n_one = 0, n_many = 0;
  for (int i = 0; i < count; ++i) {
    if (K[i] <= gemv1_max_k()) one[n_one++] = descs[i];
    else many[n_many++] = descs[i];
  }
  if (n_one > 0) {
    st = from_hip(launch_gemv1_grouped(n_one, one, w[0].quant_type, dq, bf16_out, s));
    if (st != NF4_OK) return st;
  }
  if (n_many > 0)
    st = from_hip(launch_gemv_grouped(n_many, many, 1, w[0].quant_type, dq, bf16_out, s));
  return st;
}

nf4_status nf4_gemv_grouped(int32_t count, const void *const *x_bf16, int32_t M,
                            const nf4_qweight *w, const int32_t *N, const int32_t *K,
                            int32_t compute_dtype, int32_t out_dtype, void *const *y,
                            void *stream) {
  return gemv_grouped_impl(count, x_bf16, M, w, N, K, nullptr, compute_dtype, out_dtype, y, stream);
}

static nf4_status gemm_impl(const void *x_bf16, int32_t M, const nf4_qweight *w, int32_t N,
                            int32_t K, const void *bias, int32_t compute_dtype, int32_t out_dtype,
                            void *y, void *stream) {
  ScaleArgs sc;
  nf4_status st = check_product(x_bf16, M, w, N, K, compute_dtype, out_dtype, y, &sc);
  if (st != NF4_OK) return st;
  if ((reinterpret_cast<uintptr_t>(bias) & 1u) != 0) return NF4_ERR_MISALIGNED;
  // a tile's offsets into x, the codes and y are 32-bit
  if (K > (1 << 22) || N > (1 << 21)) return NF4_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return NF4_OK;
  st = check_device();
  if (st != NF4_OK) return st;
  return from_hip(launch_gemm(static_cast<const uint16_t *>(x_bf16), M, w->packed, N, K,
                              w->blocksize, w->quant_type, sc, out_dtype == NF4_DTYPE_BF16, y,
                              static_cast<const uint16_t *>(bias),
                              reinterpret_cast<hipStream_t>(stream)));
}

nf4_status nf4_gemm(const void *x_bf16, int32_t M, const nf4_qweight *w, int32_t N, int32_t K,
                    int32_t compute_dtype, int32_t out_dtype, void *y, void *stream) {
  return gemm_impl(x_bf16, M, w, N, K, nullptr, compute_dtype, out_dtype, y, stream);
}

nf4_status nf4_linear(const void *x_bf16, int32_t M, const nf4_qweight *w, int32_t N, int32_t K,
                      const void *bias_bf16, int32_t compute_dtype, int32_t out_dtype, void *y,
                      void *stream) {
  // decode shapes take the GEMV kernels, larger batches the prefill GEMM
  if (M >= 0 && M <= NF4_GEMV_MAX_M)
    return gemv_grouped_impl(1, &x_bf16, M, w, &N, &K, &bias_bf16, compute_dtype, out_dtype, &y,
                             stream);
  return gemm_impl(x_bf16, M, w, N, K, bias_bf16, compute_dtype, out_dtype, y, stream);
}

}  // extern "C"
