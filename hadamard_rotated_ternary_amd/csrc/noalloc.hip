// The H-BitLinear forward without allocation: its scratch is a static device
// array instead of a caller-provided workspace, for callers that cannot
// allocate device memory.
#include <hip/hip_runtime.h>
#include <mutex>

#include "launch.h"

// One copy per device, held for the life of the process.  In host code the
// name `scratch` is only a stand-in for the symbol: its device address comes
// from hipGetSymbolAddress, per device, and only that address reaches the
// kernels.
static __device__ __align__(256) uint8_t scratch[HBL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device (nullptr on failure)

// The current device's copy of the array, looked up once per device with
// that device current.
hbl_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HBL_ERR_DEVICE;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_scratch[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess ? p : nullptr;
  });
  *out = g_scratch[dev];
  return *out ? HBL_OK : HBL_ERR_DEVICE;
}

}  // namespace

extern "C" hbl_status hbl_forward_noalloc(int bits, const void* x, hbl_dtype x_dtype, const float* gain,
                                          const uint8_t* w_packed, const float* w_alpha, int64_t M, int64_t K,
                                          int64_t N, void* y, hbl_dtype y_dtype, hipStream_t stream) {
  // every argument check, and the size check, before anything touches the device
  if (hbl_status s = hbl::forward_check(bits, x, x_dtype, gain, w_packed, w_alpha, M, K, N, y, y_dtype)) return s;
  if (M == 0) return HBL_OK;
  const size_t need = hbl_workspace_bytes(bits == 8 ? HBL_OP_FORWARD_INT8 : HBL_OP_FORWARD_INT4, M, K, N);
  if (need > HBL_NOALLOC_SCRATCH_BYTES) return HBL_ERR_SCRATCH;
  void* ws = nullptr;
  if (hbl_status s = scratch_address(&ws)) return s;
  return bits == 8 ? hbl_forward_int8(x, x_dtype, gain, w_packed, w_alpha, M, K, N, y, y_dtype, ws,
                                      HBL_NOALLOC_SCRATCH_BYTES, stream)
                   : hbl_forward_int4(x, x_dtype, gain, w_packed, w_alpha, M, K, N, y, y_dtype, ws,
                                      HBL_NOALLOC_SCRATCH_BYTES, stream);
}
