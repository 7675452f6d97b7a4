// Host-side helpers for the libwq entry points: error state, argument
// checks, device check and launch-status mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq.h"

namespace wq {

// Records the detail text for the calling thread and returns `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// WQ_OK when the current device is a gfx950; otherwise WQ_ERR_DEVICE with
// the detail recorded.  The answer is cached per device id (thread-safe).
int check_device();

// Maps the state after a launch to WQ_OK / WQ_ERR_LAUNCH.
int launch_status(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Devices the per-device host caches track (device ids 0 .. kMaxDevices-1).
constexpr int kMaxDevices = 64;

// Number of workgroups a kernel can keep resident on the whole current
// device at the given block size (occupancy query, cached per device,
// kernel and block size; safe to call from several host threads).
int resident_groups(const void* kernel, int block_threads);

// Balanced grid: the fewest workgroups that still fill `resident` slots,
// with every workgroup given the same number of batches (+-1).
inline int64_t balanced_grid(int64_t batches, int64_t resident) {
  if (batches <= 0) return 0;
  if (resident < 1) resident = 1;
  int64_t per = (batches + resident - 1) / resident;
  return (batches + per - 1) / per;
}

}  // namespace wq
