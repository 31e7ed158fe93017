// Error reporting and device checks shared by every entry point.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "common.h"

namespace ifp4 {

static thread_local char g_msg[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_msg[0] = '\0'; }

// Arch of each device, looked up once (hipGetDeviceProperties is slow).
static constexpr int kMaxDevices = 64;
static int g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
static char g_arch_name[kMaxDevices][64];
static std::mutex g_arch_mu;

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(INDEXER_FP4_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(INDEXER_FP4_EARCH, "device index %d out of range", dev);
  if (g_arch_ok[dev] == 0) {
    std::lock_guard<std::mutex> lock(g_arch_mu);
    if (g_arch_ok[dev] == 0) {
      hipDeviceProp_t prop;
      e = hipGetDeviceProperties(&prop, dev);
      if (e != hipSuccess) return fail(INDEXER_FP4_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
      snprintf(g_arch_name[dev], sizeof g_arch_name[dev], "%s", prop.gcnArchName);
      g_arch_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
  }
  if (g_arch_ok[dev] != 1)
    return fail(INDEXER_FP4_EARCH, "device %d is %s; this library runs on gfx950 only", dev, g_arch_name[dev]);
  return INDEXER_FP4_OK;
}

int launch_status(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(INDEXER_FP4_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return INDEXER_FP4_OK;
}

}  // namespace ifp4

extern "C" const char *indexer_fp4_last_error(void) { return ifp4::g_msg; }
extern "C" const char *indexer_last_error(void) { return ifp4::g_msg; }
