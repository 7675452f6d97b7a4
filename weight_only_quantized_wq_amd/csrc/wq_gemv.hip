// Batch-1 (and small-M) decode matvecs y = x . W^T over bf16, int8 per-row
// and int4 G=32 weights, streamed from HBM: launch planning and the C entry
// points.  The kernel itself is in wq_gemv_kernel.hpp.
#include <stdint.h>

#include "wq_gemv_kernel.hpp"
#include "wq_host.hpp"

namespace wq {

// ---------------------------------------------------------------------------
// Host side: plan selection and launch.

using LaunchFn = int (*)(const GemvArgs&, int threads, hipStream_t);

template <class F, int M, int CPL, int U, int WAVES, bool PF>
int launch_one(const GemvArgs& a0, int threads, hipStream_t stream) {
  static int resident = 0;
  auto kern = gemv_kernel<F, M, CPL, U, WAVES, PF>;
  if (resident == 0) resident = resident_groups(reinterpret_cast<const void*>(kern), threads);
  GemvArgs a = a0;
  int64_t grid = balanced_grid(a.batches, resident);
  if (grid <= 0) return WQ_OK;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, stream, a);
  return launch_status("gemv");
}

constexpr int kU = 2;

// Candidate (chunks-per-lane, waves-per-workgroup) plans per format.  A lane
// holds CPL chunks of activations in registers; split = ceil(chunks / (64
// CPL)) waves share a row.
template <class F, int M>
struct Plans;

#define WQ_PLAN(CPL, WAVES) {CPL, WAVES, &launch_one<F, M, CPL, kU, WAVES, false>}
struct PlanEntry {
  int cpl;
  int waves;
  LaunchFn fn;
};

// A workgroup of 4 waves may use up to 512 VGPRs per lane, one of 8 waves
// 256 and one of 16 waves 128; plans are listed only where the kernel fits
// its workgroup size without spilling.
template <>
struct Plans<FmtBf16, 1> {
  using F = FmtBf16;
  static constexpr int M = 1;
  static constexpr PlanEntry list[] = {WQ_PLAN(8, 4), WQ_PLAN(7, 4), WQ_PLAN(6, 4), WQ_PLAN(4, 4),
                                       WQ_PLAN(2, 4), WQ_PLAN(8, 8), WQ_PLAN(7, 8), WQ_PLAN(6, 8),
                                       WQ_PLAN(8, 16)};
};
template <>
struct Plans<FmtInt8, 1> {
  using F = FmtInt8;
  static constexpr int M = 1;
  static constexpr PlanEntry list[] = {WQ_PLAN(4, 4), WQ_PLAN(6, 4), WQ_PLAN(7, 4), WQ_PLAN(2, 4),
                                       WQ_PLAN(1, 4), WQ_PLAN(4, 8), WQ_PLAN(6, 8), WQ_PLAN(7, 8),
                                       WQ_PLAN(4, 16)};
};
template <>
struct Plans<FmtInt4, 1> {
  using F = FmtInt4;
  static constexpr int M = 1;
  static constexpr PlanEntry list[] = {WQ_PLAN(2, 4), WQ_PLAN(4, 4), WQ_PLAN(6, 4), WQ_PLAN(7, 4),
                                       WQ_PLAN(1, 4), WQ_PLAN(4, 8), WQ_PLAN(7, 8), WQ_PLAN(8, 8),
                                       WQ_PLAN(2, 16)};
};
// speculative-verify rows: the activations of all M tokens stay in registers
#define WQ_SMALLM_PLANS(MM, ...)                                             \
  template <>                                                                \
  struct Plans<FmtInt4, MM> {                                                \
    using F = FmtInt4;                                                       \
    static constexpr int M = MM;                                             \
    static constexpr PlanEntry list[] = {__VA_ARGS__};                       \
  };
WQ_SMALLM_PLANS(2, WQ_PLAN(1, 4), WQ_PLAN(2, 4), WQ_PLAN(2, 8), WQ_PLAN(4, 8), WQ_PLAN(1, 16))
WQ_SMALLM_PLANS(3, WQ_PLAN(1, 4), WQ_PLAN(2, 4), WQ_PLAN(2, 8), WQ_PLAN(1, 16))
WQ_SMALLM_PLANS(4, WQ_PLAN(1, 4), WQ_PLAN(2, 4), WQ_PLAN(2, 8), WQ_PLAN(1, 16))
WQ_SMALLM_PLANS(5, WQ_PLAN(1, 4), WQ_PLAN(1, 8), WQ_PLAN(2, 8))
WQ_SMALLM_PLANS(6, WQ_PLAN(1, 4), WQ_PLAN(1, 8))
WQ_SMALLM_PLANS(7, WQ_PLAN(1, 4), WQ_PLAN(1, 8))
WQ_SMALLM_PLANS(8, WQ_PLAN(1, 4), WQ_PLAN(1, 8))
#undef WQ_SMALLM_PLANS
#undef WQ_PLAN

// Picks the plan covering `chunks` with the fewest idle lanes; ties go to the
// plan with fewer waves per row (less cross-wave reduction), then to fewer
// registers.  Returns false when no plan covers the row.
template <class F, int M>
bool choose_plan(int64_t chunks, PlanEntry& best, int& split) {
  bool found = false;
  int64_t best_waste = 0;
  int best_split = 0;
  for (const PlanEntry& p : Plans<F, M>::list) {
    int64_t per_wave = (int64_t)kWave * p.cpl;
    int64_t s = chunks == 0 ? 1 : (chunks + per_wave - 1) / per_wave;
    if (s > p.waves) continue;
    int64_t waste = s * per_wave - chunks;
    bool better = !found || waste < best_waste ||
                  (waste == best_waste && (s < best_split || (s == best_split && p.cpl < best.cpl)));
    if (better) {
      found = true;
      best = p;
      best_waste = waste;
      best_split = (int)s;
    }
  }
  split = best_split;
  return found;
}

template <class F, int M>
int run_gemv(GemvArgs a, hipStream_t stream, const char* name) {
  PlanEntry p{};
  int split = 0;
  if (!choose_plan<F, M>(a.chunks, p, split))
    return fail(WQ_ERR_SHAPE, "%s: k = %lld is larger than the largest supported row", name, (long long)a.k);
  int groups = p.waves / split;
  a.split = split;
  a.groups = groups;
  int64_t rows_per_batch = (int64_t)groups * kU;
  a.batches = (a.n + rows_per_batch - 1) / rows_per_batch;
  return p.fn(a, split * groups * kWave, stream);
}

// Host checks in a fixed order -- null pointers, then sizes, then alignment --
// so a call is rejected for the first problem in that order.  `aux` is the
// scale (int8) or scale/zero (int4) array, checked when `need_aux`.
static int check_common(const char* name, const void* x, const void* w, const void* aux, bool need_aux, int64_t n,
                        int64_t k, const float* y32, const uint16_t* y16, int kmult, int64_t m = 1) {
  if (!x || !w) return fail(WQ_ERR_NULL, "%s: x and the weights must be non-null", name);
  if (need_aux && !aux) return fail(WQ_ERR_NULL, "%s: the scale array must be non-null", name);
  if (!y32 && !y16) return fail(WQ_ERR_NULL, "%s: at least one of y_f32 / y_bf16 must be non-null", name);
  if (n < 0 || k < 0) return fail(WQ_ERR_SHAPE, "%s: negative size (n = %lld, k = %lld)", name, (long long)n, (long long)k);
  if (k % kmult != 0) return fail(WQ_ERR_SHAPE, "%s: k = %lld is not a multiple of %d", name, (long long)k, kmult);
  if (m < 1 || m > 8) return fail(WQ_ERR_SHAPE, "%s: m = %lld outside [1, 8]", name, (long long)m);
  if (n > ((int64_t)1 << 31)) return fail(WQ_ERR_SHAPE, "%s: n = %lld too large", name, (long long)n);
  if (k > ((int64_t)1 << 24)) return fail(WQ_ERR_SHAPE, "%s: k = %lld too large", name, (long long)k);
  if (!aligned16(x) || !aligned16(w)) return fail(WQ_ERR_ALIGN, "%s: x and weights must be 16-byte aligned", name);
  return WQ_OK;
}

}  // namespace wq

using namespace wq;

extern "C" int wq_gemv_bf16(const uint16_t* x, const uint16_t* w, int64_t n, int64_t k, float* y_f32,
                            uint16_t* y_bf16, void* stream) {
  int rc = check_common("wq_gemv_bf16", x, w, nullptr, false, n, k, y_f32, y_bf16, 8);
  if (rc) return rc;
  if (n == 0) return WQ_OK;
  if ((rc = check_device())) return rc;
  GemvArgs a{};
  a.x = x;
  a.w = reinterpret_cast<const uint8_t*>(w);
  a.y32 = y_f32;
  a.y16 = y_bf16;
  a.n = n;
  a.k = k;
  a.row_bytes = 2 * k;
  a.chunks = (int32_t)(k / 8);
  return run_gemv<FmtBf16, 1>(a, (hipStream_t)stream, "wq_gemv_bf16");
}

extern "C" int wq_gemv_int8(const uint16_t* x, const int8_t* q, const uint16_t* scale, int64_t n, int64_t k,
                            float* y_f32, uint16_t* y_bf16, void* stream) {
  int rc = check_common("wq_gemv_int8", x, q, scale, true, n, k, y_f32, y_bf16, 16);
  if (rc) return rc;
  if (n == 0) return WQ_OK;
  if ((rc = check_device())) return rc;
  GemvArgs a{};
  a.x = x;
  a.w = reinterpret_cast<const uint8_t*>(q);
  a.scale = scale;
  a.y32 = y_f32;
  a.y16 = y_bf16;
  a.n = n;
  a.k = k;
  a.row_bytes = k;
  a.chunks = (int32_t)(k / 16);
  return run_gemv<FmtInt8, 1>(a, (hipStream_t)stream, "wq_gemv_int8");
}

static int int4_args(const char* name, const uint16_t* x, const uint8_t* qpacked, const uint16_t* sz, int64_t n,
                     int64_t k, float* y_f32, uint16_t* y_bf16, GemvArgs& a, int64_t m = 1) {
  int rc = check_common(name, x, qpacked, sz, true, n, k, y_f32, y_bf16, 32, m);
  if (rc) return rc;
  if ((reinterpret_cast<uintptr_t>(sz) & 3u) != 0) return fail(WQ_ERR_ALIGN, "%s: sz must be 4-byte aligned", name);
  a = GemvArgs{};
  a.x = x;
  a.w = qpacked;
  a.sz = reinterpret_cast<const uint32_t*>(sz);
  a.y32 = y_f32;
  a.y16 = y_bf16;
  a.n = n;
  a.k = k;
  a.row_bytes = k / 2;
  a.chunks = (int32_t)(k / 32);
  return WQ_OK;
}

extern "C" int wq_gemv_int4g32(const uint16_t* x, const uint8_t* qpacked, const uint16_t* sz, int64_t n, int64_t k,
                               float* y_f32, uint16_t* y_bf16, void* stream) {
  GemvArgs a;
  int rc = int4_args("wq_gemv_int4g32", x, qpacked, sz, n, k, y_f32, y_bf16, a);
  if (rc) return rc;
  if (n == 0) return WQ_OK;
  if ((rc = check_device())) return rc;
  return run_gemv<FmtInt4, 1>(a, (hipStream_t)stream, "wq_gemv_int4g32");
}

extern "C" int wq_gemm_smallM(const uint16_t* x, int64_t m, const uint8_t* qpacked, const uint16_t* sz, int64_t n,
                              int64_t k, float* y_f32, uint16_t* y_bf16, void* stream) {
  GemvArgs a;
  int rc = int4_args("wq_gemm_smallM", x, qpacked, sz, n, k, y_f32, y_bf16, a, m);
  if (rc) return rc;
  if (n == 0) return WQ_OK;
  if ((rc = check_device())) return rc;
  hipStream_t s = (hipStream_t)stream;
  switch (m) {
    case 1: return run_gemv<FmtInt4, 1>(a, s, "wq_gemm_smallM");
    case 2: return run_gemv<FmtInt4, 2>(a, s, "wq_gemm_smallM");
    case 3: return run_gemv<FmtInt4, 3>(a, s, "wq_gemm_smallM");
    case 4: return run_gemv<FmtInt4, 4>(a, s, "wq_gemm_smallM");
    case 5: return run_gemv<FmtInt4, 5>(a, s, "wq_gemm_smallM");
    case 6: return run_gemv<FmtInt4, 6>(a, s, "wq_gemm_smallM");
    case 7: return run_gemv<FmtInt4, 7>(a, s, "wq_gemm_smallM");
    default: return run_gemv<FmtInt4, 8>(a, s, "wq_gemm_smallM");
  }
}
