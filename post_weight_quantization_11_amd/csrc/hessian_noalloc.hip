// The Hessian accumulation for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the token-split partial sums live in a static device array of
// GPTQ_HESSIAN_NOALLOC_SCRATCH_BYTES bytes instead of a caller workspace.
//
// In host code `scratch` names a host-side stand-in of the array, not its
// device address: the address is looked up once per device with
// hipGetSymbolAddress and only that pointer is handed to kernels.  Every
// device holds its own copy of the array for the rest of the process; calls
// on one device share it, so calls that overlap on one device race.  Nothing
// in it needs clearing between calls: every partial tile a pass reads was
// written by the same pass.
#include <mutex>

#include "common.h"
#include "hessian_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[GPTQ_HESSIAN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// The device address of this device's scratch array (nullptr on failure).
void* scratch_ptr(int dev) {
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  return g_ptr[dev];
}

}  // namespace

extern "C" gptq_status gptq_hessian_accumulate_noalloc(float* H, int64_t n, const void* X, int x_dtype,
                                                       int64_t tokens, int64_t ldx, float alpha, int reset,
                                                       void* stream) {
  if (n < 0 || tokens < 0 || !gptq::valid_dtype(x_dtype)) return GPTQ_ERR_INVALID_ARG;
  if (n > 0 && gptq::hessian_split_bytes(n) > (int64_t)GPTQ_HESSIAN_NOALLOC_SCRATCH_BYTES)
    return GPTQ_ERR_UNSUPPORTED;
  if (n == 0) return GPTQ_OK;
  if (H == nullptr || (tokens > 0 && (X == nullptr || ldx < n))) return GPTQ_ERR_INVALID_ARG;
  int dev = 0;
  GPTQ_TRY_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return GPTQ_ERR_UNSUPPORTED;
  void* ws = scratch_ptr(dev);
  if (ws == nullptr) return GPTQ_ERR_HIP;
  return gptq::hessian_accumulate_bounded(H, n, X, x_dtype, tokens, ldx, alpha, reset, ws,
                                          (size_t)GPTQ_HESSIAN_NOALLOC_SCRATCH_BYTES, stream);
}
