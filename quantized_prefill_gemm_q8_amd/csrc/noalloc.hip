// qgemm_prefill_noalloc: qgemm_prefill for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The activation workspace lives in a file-scope
// device array of fixed size instead of a caller buffer; the kernels are
// qgemm_prefill's, reading that array through its device address.
//
// The array's name is a host-side stand-in in host code, not a device
// address: the address is looked up once per device (hipGetSymbolAddress,
// with that device current) on the entry point's first call there and kept,
// and only that address is ever handed to kernels.
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "common.h"

// Each device holds its own copy for the life of the process.
static __device__ __align__(256) uint8_t scratch[QG_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's copy of `scratch` (nullptr on failure).
void* scratch_ptr(int dev) {
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace

extern "C" int qgemm_prefill_noalloc(const void* q_weights, int fmt, const void* x, int x_dtype, int64_t M,
                                     int64_t N, int64_t K, float* y, void* stream) {
  // every argument rule of qgemm_prefill except the workspace's, which the
  // scratch replaces; sizes beyond the scratch are refused before any launch
  if (!q_weights || !x || !y || M < 1 || N < 1 || K < 256 || K % 256 != 0) return QG_EINVAL;
  const size_t need = qgemm_workspace_bytes(M, K);
  if (need == 0) return QG_EINVAL;
  if (need > static_cast<size_t>(QG_NOALLOC_SCRATCH_BYTES)) return QG_ENOSCRATCH;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QG_EDEVICE;
  void* ws = scratch_ptr(dev);
  if (!ws) return QG_ELAUNCH;
  return qgemm_prefill(q_weights, fmt, x, x_dtype, M, N, K, y, ws, static_cast<size_t>(QG_NOALLOC_SCRATCH_BYTES),
                       stream);
}
