// status.cpp -- status strings and the thread-local error detail.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>

#include "tg_common.hpp"

namespace {
thread_local char g_last_error[512] = "";
}

namespace tg {

tg_status fail(tg_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_last_error[0] = '\0'; }

int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];   // 0: not read yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;
  cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

tg_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(TG_ERR_LAUNCH, "%s: kernel launch failed: %s", what,
                hipGetErrorString(e));
  clear_error();
  return TG_OK;
}

}  // namespace tg

extern "C" const char* tg_status_str(int status) {
  switch (status) {
    case TG_OK: return "TG_OK";
    case TG_ERR_INVALID_ARGUMENT: return "TG_ERR_INVALID_ARGUMENT";
    case TG_ERR_UNSUPPORTED: return "TG_ERR_UNSUPPORTED";
    case TG_ERR_WORKSPACE: return "TG_ERR_WORKSPACE";
    case TG_ERR_LAUNCH: return "TG_ERR_LAUNCH";
    default: return "TG_ERR_UNKNOWN";
  }
}

extern "C" const char* tg_last_error(void) { return g_last_error; }
