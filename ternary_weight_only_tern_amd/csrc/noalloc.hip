// The decode product for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): tern_gemv with its workspace in a fixed device array of
// kScratchBytes per GPU, so the caller passes only the matrix, x and y.
//
// The array lives in the library's code object, one copy per GPU the
// library runs on, for the life of the process.  Its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and kept; host code uses only that address.  Every call on a GPU shares
// the GPU's array and finds the previous call's contents there: the product
// clears what it needs cleared inside its own launch sequence, and calls that
// overlap in time on one GPU race on the array.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <mutex>

#include "internal.h"
#include "tern.h"

namespace {

constexpr size_t kScratchBytes = TERN_NOALLOC_WORKSPACE_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (looked up on the device's first
// call), or NULL with the error recorded.
void* device_scratch(tern_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = tern::record_failure(TERN_E_HIP, "tern_gemv_noalloc: hipGetDevice failed");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *st = tern::record_failure(TERN_E_UNSUPPORTED, "tern_gemv_noalloc: device index beyond the 64 it tracks");
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[160];
      std::snprintf(msg, sizeof(msg), "tern_gemv_noalloc: hipGetSymbolAddress(scratch) failed: %s",
                    hipGetErrorString(e));
      *st = tern::record_failure(TERN_E_HIP, msg);
      return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" tern_status tern_gemv_noalloc(const tern_matrix* w, const uint16_t* x, int32_t m, void* y,
                                         int32_t y_dtype, void* stream) {
  if (!w) return tern::record_failure(TERN_E_INVAL, "tern_gemv_noalloc: matrix is NULL");
  const size_t need = tern_workspace_bytes(w, m);
  if (need > kScratchBytes) {
    char msg[200];
    std::snprintf(msg, sizeof(msg),
                  "tern_gemv_noalloc: this product needs %zu workspace bytes, more than the %zu of its fixed "
                  "array (use tern_gemv with a workspace)", need, kScratchBytes);
    return tern::record_failure(TERN_E_WORKSPACE, msg);
  }
  tern_status st = TERN_OK;
  void* ws = device_scratch(&st);
  if (!ws) return st;
  return tern_gemv(w, x, m, y, y_dtype, ws, kScratchBytes, stream);
}
