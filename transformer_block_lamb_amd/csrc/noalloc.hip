// lamb_step_noalloc: lamb_step with its scratch in a static device array
// instead of a caller buffer, for callers that cannot allocate device memory
// (code under graph capture, tight loops, harnesses that forbid allocation).
//
// The scratch of a LAMB step is the per-workgroup partial sums of ||w||^2
// and ||u||^2 and the per-tensor trust ratios.  Nothing in it has to start
// at zero: pass A writes every partial before the finalize kernel reads it,
// and the finalize writes every ratio before pass B reads it.  Each device
// holds its own copy of the array until the process ends; its device
// address is looked up once per device, with that device current, and kept.
// Every call on one device shares that device's array, so calls that
// overlap on one device (two streams, two threads) race; callers order them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/ptb.h"

namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)2 << 20;  // 2 MiB
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of the current device's copy of `scratch`.  (In host
// code the array's name is only a host-side stand-in; it is never handed to
// a kernel or a copy.)
int scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PTB_ERR_HIP;
  if (stream != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return PTB_ERR_INVALID_ARG;
    if (sdev != dev) return PTB_ERR_INVALID_ARG;  // the stream's device must be current
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PTB_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return PTB_OK;
}

}  // namespace

extern "C" {

size_t lamb_noalloc_max_scratch_bytes(void) { return kNoAllocScratchBytes; }

int lamb_step_noalloc(const lamb_tensor* tensors, int32_t n_tensors, float lr, float beta1,
                      float beta2, float eps, int64_t step, float* ratios_out,
                      hipStream_t stream) {
  const size_t need = lamb_scratch_bytes(tensors, n_tensors);
  if (need == 0) return PTB_ERR_INVALID_ARG;
  if (need > kNoAllocScratchBytes) return PTB_ERR_WORKSPACE;
  void* ws = nullptr;
  const int st = scratch_address(stream, &ws);
  if (st != PTB_OK) return st;
  // lamb_step validates every other argument before it launches anything
  return lamb_step(tensors, n_tensors, lr, beta1, beta2, eps, step, ratios_out, ws,
                   kNoAllocScratchBytes, stream);
}

}  // extern "C"
