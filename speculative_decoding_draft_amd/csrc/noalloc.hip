// eagle_op_linear_noalloc (include/eagle_ops.h): the projection of
// eagle_op_linear with its split-K partial planes in a fixed device array of
// this library instead of a caller workspace, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops).
#include <hip/hip_runtime.h>

#include <mutex>

#include "eagle_ops.h"

namespace {

// The array every call on a device uses for the partial planes. Each device
// the library runs on holds its own copy until the process ends.
static __device__ __align__(256) unsigned char scratch[EAGLE_OP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];   // device address of `scratch`, per device
std::mutex g_mu;

// Device address of this device's copy of `scratch`, looked up once per
// device with that device current. The array's name in host code is only a
// host-side handle: kernels must get this address instead.
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" eagle_status eagle_op_linear_noalloc(int32_t dtype, int32_t epilogue, const void* x,
                                                const void* w, void* y, int32_t M, int32_t N,
                                                int32_t K, void* stream) {
  if (!x || !w || !y) return EAGLE_E_INVALID;
  // 0 for a bad shape too: eagle_op_linear then rejects it before any launch
  const uint64_t need = eagle_op_linear_workspace(dtype, epilogue, M, N, K);
  if (need > EAGLE_OP_NOALLOC_SCRATCH_BYTES) return EAGLE_E_CAPACITY;
  void* ws = nullptr;
  if (scratch_ptr(&ws) != hipSuccess) return EAGLE_E_HIP;
  return eagle_op_linear(dtype, epilogue, x, w, y, M, N, K, ws, EAGLE_OP_NOALLOC_SCRATCH_BYTES,
                         stream);
}
