// libwq: status strings, thread-local error text, device checks.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "wq_host.hpp"

namespace wq {

static thread_local char t_err[512];

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(t_err, sizeof(t_err), fmt, ap);
  va_end(ap);
  return status;
}

int check_device() {
  // 0 = unknown, 1 = gfx950, 2 = other
  static int verdict[64] = {0};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(WQ_ERR_DEVICE, "no current HIP device (%s)", hipGetErrorString(e));
  }
  if (dev < 64 && verdict[dev] == 1) return WQ_OK;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(WQ_ERR_DEVICE, "hipGetDeviceProperties(%d) failed: %s", dev, hipGetErrorString(e));
  }
  bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) verdict[dev] = ok ? 1 : 2;
  if (!ok) return fail(WQ_ERR_DEVICE, "device %d is %s; libwq is built for gfx950 only", dev, prop.gcnArchName);
  return WQ_OK;
}

int launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WQ_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return WQ_OK;
}

int resident_groups(const void* kernel, int block_threads) {
  int dev = 0;
  (void)hipGetDevice(&dev);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, 0) != hipSuccess ||
      per_cu < 1) {
    (void)hipGetLastError();
    per_cu = 1;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
    (void)hipGetLastError();
    cus = 256;
  }
  return per_cu * cus;
}

}  // namespace wq

extern "C" const char* wq_status_string(int status) {
  switch (status) {
    case WQ_OK: return "ok";
    case WQ_ERR_NULL: return "null pointer";
    case WQ_ERR_SHAPE: return "unsupported or inconsistent size";
    case WQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case WQ_ERR_DEVICE: return "no gfx950 device";
    case WQ_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" const char* wq_last_error(void) { return wq::t_err; }
