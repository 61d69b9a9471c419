// nf4_noalloc.hip -- nf4_linear_noalloc, the linear layer for callers that
// cannot allocate device memory (code under stream capture, serving loops,
// harnesses that forbid allocation): nf4_linear_ws with its workspace in a
// static device array instead of a caller's buffer.
//
// The array is a file-scope __device__ object, so every device the library
// runs on holds its own copy until the process ends. Host code never uses
// the array's name as an address: on the first call on a device, with that
// device current, hipGetSymbolAddress gives that device's copy, and the
// pointer is kept per device and passed to the kernels like any workspace.
#include <mutex>

#include "nf4_internal.h"

namespace {

constexpr size_t kScratchBytes = NF4_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void *g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// The current device's copy of `scratch` (looked up once per device).
nf4_status current_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NF4_ERR_DEVICE;
  std::call_once(g_scratch_once[dev], [dev] {
    void *p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch[dev] == nullptr) return NF4_ERR_DEVICE;
  *out = g_scratch[dev];
  return NF4_OK;
}

}  // namespace

extern "C" nf4_status nf4_linear_noalloc(const void *x, int64_t ldx, int32_t M,
                                         const nf4_qweight *w, int32_t N, int32_t K,
                                         const void *bias, int32_t compute_dtype,
                                         int32_t out_dtype, void *y, int64_t ldy, void *stream) {
  if (w == nullptr) return NF4_ERR_INVALID_ARGUMENT;
  // decode products take their K split from the scratch; prefill products the
  // fused GEMM (their dequantized weight would not fit)
  const int64_t need = M <= NF4_GEMV_MAX_M
                           ? nf4::linear_workspace_bytes(M, N, K, w->blocksize, compute_dtype,
                                                         out_dtype, w->double_quant)
                           : 0;
  if (need > (int64_t)kScratchBytes) return NF4_ERR_SCRATCH;
  void *ws = nullptr;
  if (need > 0) {
    const nf4_status st = current_scratch(&ws);
    if (st != NF4_OK) return st;
  }
  return nf4::linear_with_workspace(x, ldx, M, w, N, K, bias, compute_dtype, out_dtype, y, ldy,
                                    ws, ws != nullptr ? (int64_t)kScratchBytes : 0, stream);
}
