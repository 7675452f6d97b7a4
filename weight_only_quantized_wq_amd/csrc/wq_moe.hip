// Top-2 MoE decode step for one token with int8 per-row experts (Mixtral
// 8x7B shape), as two streaming launches on the caller's stream:
//
//   1. moe_w13_kernel: every workgroup routes (softmax top-2 of the logits,
//      equal logits -> lower index; gates renormalised over the pair), then
//      streams rows j and j + f of W13 for each selected expert and writes
//      a[slot][j] = silu(h_j) * h_{j+f} (fp32) to the caller's workspace
//      (moe_top2_gemv_noalloc: to a static device array).
//   2. moe_w2_kernel: two wave teams per workgroup, one per selected expert,
//      stream row n of their expert's W2 against that expert's a; the
//      workgroup combines y[n] = g_a o_a[n] + g_b o_b[n].
//
// Only the selected experts' weights are read and no host synchronisation is
// needed: the routing decision is recomputed (identically) on the device by
// every workgroup from the 8 logits.
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "wq_host.hpp"
#include "wq_moe_kernel.hpp"

namespace wq {

// ---------------------------------------------------------------------------
// Host side

template <class K>
static int launch_grid(K kern, const MoeArgs& a, int threads, hipStream_t stream) {
  const int resident = resident_groups(reinterpret_cast<const void*>(kern), threads);
  int64_t grid = balanced_grid(a.batches, resident);
  if (grid <= 0) return WQ_OK;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, stream, a);
  return launch_status("moe_top2_gemv");
}

// W13 plans: CPL 4 with up to 8 waves; the team size is the split.
static int launch_w13(MoeArgs a, hipStream_t stream) {
  const int64_t per_wave = (int64_t)kWave * 4;
  int64_t s = (a.chunks + per_wave - 1) / per_wave;
  if (s < 1) s = 1;
  if (s > 8) return fail(WQ_ERR_SHAPE, "moe_top2_gemv: dim = %lld too large", (long long)a.dim);
  if (s <= 4) {
    a.split = (int)s;
    a.groups = 4 / (int)s;
    a.batches = (2 * a.f + a.groups - 1) / a.groups;
    return launch_grid(moe_w13_kernel<4, 4, false>, a, a.split * a.groups * kWave, stream);
  }
  a.split = (int)s;
  a.groups = 8 / (int)s;
  a.batches = (2 * a.f + a.groups - 1) / a.groups;
  return launch_grid(moe_w13_kernel<4, 8, false>, a, a.split * a.groups * kWave, stream);
}

// W2 plans: two teams of `split` waves; chunks per lane 7 (two waves per
// team cover 14336 inputs exactly) or 4.
static int launch_w2(MoeArgs a, hipStream_t stream) {
  const int64_t c = a.chunks;
  const int64_t s7 = (c + 64 * 7 - 1) / (64 * 7);
  const int64_t s4 = (c + 64 * 4 - 1) / (64 * 4);
  const int64_t waste7 = s7 * 64 * 7 - c, waste4 = s4 * 64 * 4 - c;
  if (s7 <= 2 && waste7 <= waste4) {
    // one row per team per batch, the next batch prefetched (timed best on
    // the Mixtral 8x7B shape, f = 14336)
    a.split = (int)(s7 < 1 ? 1 : s7);
    a.groups = 2;
    a.batches = a.dim;
    return launch_grid(moe_w2_kernel<7, 4, 1, true>, a, 2 * a.split * kWave, stream);
  }
  if (s4 <= 8) {
    constexpr int U = 2;
    a.split = (int)(s4 < 1 ? 1 : s4);
    a.groups = 2;
    a.batches = (a.dim + U - 1) / U;
    return launch_grid(moe_w2_kernel<4, 16, U, false>, a, 2 * a.split * kWave, stream);
  }
  return fail(WQ_ERR_SHAPE, "moe_top2_gemv: f = %lld too large", (long long)a.f);
}

}  // namespace wq

using namespace wq;

// Argument checks shared by both entry points (null -> sizes -> alignment,
// then the device).  `work` is checked only when the caller brings it.
static int moe_check(const char* name, const uint16_t* x, const float* logits, int64_t e, const int8_t* w13,
                     const uint16_t* s13, const int8_t* w2, const uint16_t* s2, int64_t dim, int64_t f,
                     const float* work, bool need_work, const float* y_f32, const uint16_t* y_bf16,
                     int64_t max_f) {
  if (!x || !logits || !w13 || !s13 || !w2 || !s2 || (need_work && !work))
    return fail(WQ_ERR_NULL, "%s: x, logits, w13, s13, w2, s2%s must be non-null", name,
                need_work ? " and work" : "");
  if (!y_f32 && !y_bf16) return fail(WQ_ERR_NULL, "%s: at least one of y_f32 / y_bf16 must be non-null", name);
  if (e != 8) return fail(WQ_ERR_SHAPE, "%s: e = %lld; only 8 experts (top-2) are supported", name, (long long)e);
  if (dim < 16 || f < 16 || dim % 16 || f % 16 || dim > 32768 || f > 32768)
    return fail(WQ_ERR_SHAPE, "%s: dim = %lld, f = %lld must be multiples of 16 in [16, 32768]", name,
                (long long)dim, (long long)f);
  if (f > max_f)
    return fail(WQ_ERR_SHAPE, "%s: f = %lld exceeds this entry point's limit of %lld (its static scratch)", name,
                (long long)f, (long long)max_f);
  if (!aligned16(x) || !aligned16(w13) || !aligned16(w2) || (need_work && !aligned16(work)))
    return fail(WQ_ERR_ALIGN, "%s: x, w13, w2%s must be 16-byte aligned", name, need_work ? " and work" : "");
  return check_device();
}

static int moe_launch(const uint16_t* x, const float* logits, int64_t e, const int8_t* w13, const uint16_t* s13,
                      const int8_t* w2, const uint16_t* s2, int64_t dim, int64_t f, float* work, float* y_f32,
                      uint16_t* y_bf16, int32_t* sel, float* gates, void* stream) {
  MoeArgs a{};
  a.x = x;
  a.logits = logits;
  a.w13 = w13;
  a.s13 = s13;
  a.w2 = w2;
  a.s2 = s2;
  a.work = work;
  a.y32 = y_f32;
  a.y16 = y_bf16;
  a.sel = sel;
  a.gates = gates;
  a.dim = dim;
  a.f = f;
  a.e = (int32_t)e;
  hipStream_t s = (hipStream_t)stream;
  a.chunks = (int32_t)(dim / 16);
  int rc = launch_w13(a, s);
  if (rc) return rc;
  a.chunks = (int32_t)(f / 16);
  return launch_w2(a, s);
}

extern "C" int moe_top2_gemv(const uint16_t* x, const float* logits, int64_t e, const int8_t* w13,
                             const uint16_t* s13, const int8_t* w2, const uint16_t* s2, int64_t dim, int64_t f,
                             float* work, float* y_f32, uint16_t* y_bf16, int32_t* sel, float* gates,
                             void* stream) {
  int rc = moe_check("moe_top2_gemv", x, logits, e, w13, s13, w2, s2, dim, f, work, true, y_f32, y_bf16, 32768);
  if (rc) return rc;
  return moe_launch(x, logits, e, w13, s13, w2, s2, dim, f, work, y_f32, y_bf16, sel, gates, stream);
}

// ---------------------------------------------------------------------------
// The same layer for callers that cannot allocate: the SwiGLU intermediate
// (fp32 [2][f]) lives in a static device array instead of a caller's
// workspace.  Each device holds its own copy of the array at its own
// address; host code never passes the array's name to a kernel (on the host
// it is a stand-in, not a device address) but the address that
// hipGetSymbolAddress returned for the current device.

constexpr int64_t kMoeScratchMaxF = 16384;    // 2 x 16384 fp32 = 128 KiB per device
static __device__ __align__(256) float scratch[2 * kMoeScratchMaxF];

static std::atomic<float*> g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

// The current device's address of `scratch`, looked up once per device (with
// that device current) and kept; null with the error recorded on failure.
static float* scratch_on_current_device(const char* name) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    fail(WQ_ERR_DEVICE, "%s: no usable current device (%d)", name, dev);
    return nullptr;
  }
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* addr = nullptr;
  e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !addr) {
    (void)hipGetLastError();
    fail(WQ_ERR_DEVICE, "%s: hipGetSymbolAddress of the static scratch failed on device %d: %s", name, dev,
         hipGetErrorString(e));
    return nullptr;
  }
  p = static_cast<float*>(addr);
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

extern "C" int moe_top2_gemv_noalloc(const uint16_t* x, const float* logits, int64_t e, const int8_t* w13,
                                     const uint16_t* s13, const int8_t* w2, const uint16_t* s2, int64_t dim,
                                     int64_t f, float* y_f32, uint16_t* y_bf16, int32_t* sel, float* gates,
                                     void* stream) {
  const char* name = "moe_top2_gemv_noalloc";
  int rc = moe_check(name, x, logits, e, w13, s13, w2, s2, dim, f, nullptr, false, y_f32, y_bf16, kMoeScratchMaxF);
  if (rc) return rc;
  float* work = scratch_on_current_device(name);
  if (!work) return WQ_ERR_DEVICE;
  // the W13 launch writes every element of work[0..2f) before the W2
  // launch (same stream) reads it: nothing needs clearing
  return moe_launch(x, logits, e, w13, s13, w2, s2, dim, f, work, y_f32, y_bf16, sel, gates, stream);
}
