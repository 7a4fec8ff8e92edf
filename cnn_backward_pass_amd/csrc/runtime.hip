// runtime.hip -- process-wide bookkeeping of libcbb.so: the HIP error text of
// the last failed launch, the launch hook (tracing), and the device error word
// that kernels raise for conditions only the data reveals (cbb_get_device_error).
#include <cstdio>
#include <mutex>

#include "cbb_internal.h"

namespace cbb {

namespace {

thread_local char g_err[512] = "";

// Launch hook: called on the calling thread after every kernel is enqueued.
std::mutex g_hook_mu;
cbb_launch_hook g_hook = nullptr;
void* g_hook_user = nullptr;

// Device error word, one per GPU: kernels OR CBB_DEVERR_* bits into it; the host
// reads and clears it in cbb_get_device_error.  Host code reaches each device's
// copy through its address, looked up once per device with that device current
// (the variable's name in host code is a stand-in, not a device address).
__device__ int32_t g_device_error;
constexpr int kMaxDevices = 64;
std::mutex g_sym_mu;
int32_t* g_device_error_ptr[kMaxDevices] = {};

}  // namespace

void set_hip_error(hipError_t e, const char* where) {
  snprintf(g_err, sizeof g_err, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

const char* last_error_text() { return g_err; }

void note_launch(const char* kernel, hipStream_t st) {
  cbb_launch_hook fn;
  void* user;
  {
    std::lock_guard<std::mutex> lk(g_hook_mu);
    fn = g_hook;
    user = g_hook_user;
  }
  if (fn) fn(user, kernel, reinterpret_cast<void*>(st));
}

int check_error(const char* where) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_hip_error(e, where);
    return CBB_EHIP;
  }
  return CBB_OK;
}

int check_launch(const char* where, hipStream_t st) {
  const int rc = check_error(where);
  if (rc == CBB_OK) note_launch(where, st);
  return rc;
}

// The current device's error word (nullptr with the HIP error recorded on failure).
int32_t* device_error_word() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_hip_error(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(g_err, sizeof g_err, "device %d beyond the %d the library tracks", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_sym_mu);
  if (!g_device_error_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_device_error));
    if (e != hipSuccess || !p) {
      set_hip_error(e, "hipGetSymbolAddress(g_device_error)");
      return nullptr;
    }
    g_device_error_ptr[dev] = static_cast<int32_t*>(p);
  }
  return g_device_error_ptr[dev];
}

}  // namespace cbb

using namespace cbb;

extern "C" {

int cbb_set_launch_hook(cbb_launch_hook fn, void* user) {
  std::lock_guard<std::mutex> lk(g_hook_mu);
  g_hook = fn;
  g_hook_user = fn ? user : nullptr;
  return CBB_OK;
}

int cbb_get_device_error(void* stream, int* code) {
  if (!code) return CBB_EINVAL;
  *code = 0;
  int32_t* word = device_error_word();
  if (!word) return CBB_EHIP;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    set_hip_error(e, "hipStreamSynchronize");
    return CBB_EHIP;
  }
  int32_t v = 0;
  const int32_t zero = 0;
  e = hipMemcpyAsync(&v, word, sizeof v, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipMemcpyAsync(word, &zero, sizeof zero, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    set_hip_error(e, "reading the device error word");
    return CBB_EHIP;
  }
  *code = v;
  return CBB_OK;
}

}  // extern "C"
