// Allocation-free form of based_layer_fwd: the segment records that the
// layered pass keeps between its kernels live in a file-scope device array
// instead of a caller workspace, for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops, harnesses that forbid
// hipMalloc).
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it only stands in for the symbol): the first call on a device, with
// that device current, takes the array's device address from
// hipGetSymbolAddress and keeps it for that device.
#include "../../include/based.h"

#include <hip/hip_runtime.h>

#include <mutex>

#define BASED_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = (size_t)BASED_NOALLOC_SCRATCH_MB << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (null: not looked up yet)

// Device address of this device's scratch array, or null on a HIP error.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

BASED_API int based_layer_fwd_noalloc(const void* q, const void* k, const void* v, float* y_lin, float* y_swa,
                                      const float* S_in, const float* z_in, float* S_out, float* z_out, int B,
                                      int H, int L, int d_k, int d_v, int window, float scale, int dtype,
                                      void* stream) {
  const size_t need = based_linattn_workspace_bytes(B, H, L, d_k, d_v, dtype);
  if (need > kScratchBytes) return BASED_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = device_scratch();
    if (!ws) return BASED_ERR_HIP;
  }
  return based_layer_fwd(q, k, v, y_lin, y_swa, S_in, z_in, S_out, z_out, B, H, L, d_k, d_v, window, scale, dtype,
                         ws, need > 0 ? kScratchBytes : 0, stream);
}
