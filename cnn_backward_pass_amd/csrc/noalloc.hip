// noalloc.hip -- cbb_conv_block_backward_noalloc: the conv block backward with
// its scratch memory in a library-owned static device array instead of a
// caller-provided workspace, for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in the code object: each GPU the library runs on holds its
// own copy (kNoAllocScratchBytes) from module load until the process ends.
// Host code never passes the array's name to a kernel -- in host code that
// name is a stand-in, not a device address -- but the address
// hipGetSymbolAddress returns for it on the current device, looked up once per
// device and kept.
#include <cstdio>
#include <mutex>

#include "cbb_internal.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[CBB_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch` (set-up on the first call per device, with that
// device current); nullptr with the HIP error recorded on failure.
void* scratch_on_current_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    cbb::set_hip_error(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    cbb::set_hip_error(hipErrorInvalidDevice, "cbb_conv_block_backward_noalloc: device index");
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      cbb::set_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol,
                         "hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int cbb_conv_block_backward_noalloc(const cbb_conv_desc* desc, const float* x, const float* w,
                                    const float* y, const float* x_norm, const float* var,
                                    const float* gamma, const float* delta, float* dz, float* dw,
                                    float* db, float* dgamma, float* dx, int dx_accumulate,
                                    void* stream) {
  size_t need = 0;
  int rc = cbb_conv_block_workspace_size(desc, &need);
  if (rc) return rc;
  if (need > (size_t)CBB_NOALLOC_SCRATCH_BYTES) return CBB_ESCRATCH;
  // every argument rule of cbb_conv_block_backward, checked before the device is touched
  rc = cbb::check_block_backward(desc, x, w, y, x_norm, var, gamma, delta, dz, dw, db, dgamma,
                                 dx, dx_accumulate);
  if (rc) return rc;
  void* ws = scratch_on_current_device();
  if (!ws) return CBB_EHIP;
  return cbb_conv_block_backward(desc, x, w, y, x_norm, var, gamma, delta, dz, dw, db, dgamma,
                                 dx, dx_accumulate, ws, (size_t)CBB_NOALLOC_SCRATCH_BYTES,
                                 stream);
}

}  // extern "C"
