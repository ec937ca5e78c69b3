// w4a8_linear_noalloc (include/w4a8.h): w4a8_linear for callers that cannot
// allocate device memory.  Its workspace (the quantised activations, their
// scales and any split-K partial sums) is a static device array that every
// GPU the library runs on holds from the library's first use on it until the
// process ends.  The call allocates and frees nothing.
#include <cstdio>
#include <mutex>

#include "../../include/w4a8.h"
#include "w4a8_internal.h"

namespace {

// The host-side name `scratch` is not a device address: host code uses only
// the per-device pointer that hipGetSymbolAddress returns for it.
static __device__ __align__(256) uint8_t scratch[W4A8_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// This device's address of `scratch`, looked up once per device (with that
// device current) and kept; null (and the error recorded) on failure.
void* scratch_for_current_device(int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    *status = w4a8::report_error(W4A8_ERR_DEVICE, "no current HIP device for the static scratch");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[160];
      snprintf(msg, sizeof msg, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
               hipGetErrorString(e));
      (void)hipGetLastError();
      *status = w4a8::report_error(W4A8_ERR_DEVICE, msg);
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int w4a8_linear_noalloc(const void* x, int32_t x_dtype, const void* packed,
                                   size_t packed_bytes, int64_t M, int64_t N, int64_t K,
                                   int32_t group, uint16_t* y, void* stream) {
  // shape and size checks first: a rejected call touches no device state
  if (w4a8_packed_weight_bytes(N, K, group) == 0)
    return w4a8::report_error(W4A8_ERR_UNSUPPORTED_SHAPE,
                              "unsupported weight shape (group 128, K % 128 == 0, N % 16 == 0)");
  if (M <= 0 || M > ((int64_t)1 << 24))
    return w4a8::report_error(W4A8_ERR_INVALID_ARG, "M out of range");
  if (!x || !y || !packed) return w4a8::report_error(W4A8_ERR_INVALID_ARG, "null pointer");
  const size_t need = w4a8_linear_workspace_bytes(M, N, K, group);
  if (need > (size_t)W4A8_NOALLOC_SCRATCH_BYTES) {
    char msg[200];
    snprintf(msg, sizeof msg,
             "M=%lld N=%lld K=%lld needs %zu bytes of workspace; the static scratch holds %zu "
             "(use w4a8_linear with a caller workspace)",
             (long long)M, (long long)N, (long long)K, need, (size_t)W4A8_NOALLOC_SCRATCH_BYTES);
    return w4a8::report_error(W4A8_ERR_BUFFER_TOO_SMALL, msg);
  }
  int status = W4A8_OK;
  void* ws = scratch_for_current_device(&status);
  if (!ws) return status;
  // Nothing in the workspace must start at zero: every path writes what it
  // later reads (codes, scales, partial sums) within the same call.
  return w4a8_linear(x, x_dtype, packed, packed_bytes, M, N, K, group, y, ws,
                     (size_t)W4A8_NOALLOC_SCRATCH_BYTES, stream);
}
