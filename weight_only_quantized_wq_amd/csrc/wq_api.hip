// libwq: status strings, thread-local error text, device checks and the
// per-device occupancy cache.  The host-side caches are safe to use from
// several host threads at once and are keyed by device id.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

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

// Per-device verdict of check_device: 0 = unknown, 1 = gfx950, 2 = other.
// Every thread that asks computes the same answer, so a relaxed store of it
// races with nothing.
static std::atomic<int> g_verdict[kMaxDevices];

int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(WQ_ERR_DEVICE, "no current HIP device (%s)", hipGetErrorString(e));
  }
  if (dev < kMaxDevices && g_verdict[dev].load(std::memory_order_relaxed) == 1) return WQ_OK;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(WQ_ERR_DEVICE, "hipGetDeviceProperties(%d) failed: %s", dev, hipGetErrorString(e));
  }
  bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_verdict[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  if (!ok) return fail(WQ_ERR_DEVICE, "device %d is %s; libwq is built for gfx950 only", dev, prop.gcnArchName);
  return WQ_OK;
}

int launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WQ_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return WQ_OK;
}

static int query_resident(int dev, const void* kernel, int block_threads) {
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

// (device, kernel, block size) -> resident workgroups; filled on first use
// under the lock, so concurrent first calls on any devices are safe.
static std::mutex g_resident_mu;
static std::map<std::tuple<int, const void*, int>, int> g_resident;

int resident_groups(const void* kernel, int block_threads) {
  int dev = 0;
  (void)hipGetDevice(&dev);
  const auto key = std::make_tuple(dev, kernel, block_threads);
  std::lock_guard<std::mutex> lock(g_resident_mu);
  auto it = g_resident.find(key);
  if (it != g_resident.end()) return it->second;
  const int r = query_resident(dev, kernel, block_threads);
  g_resident.emplace(key, r);
  return r;
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
