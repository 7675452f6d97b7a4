// Whole decode step in one launch: plan once on the host, then launch the
// persistent step kernel (wq_gemv_kernel.hpp) as often as needed.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "wq_gemv_kernel.hpp"
#include "wq_host.hpp"
#include "wq_step_shared.hpp"
#include "wq_verify.hpp"

namespace wq {

// One persistent kernel configuration per (format, tokens per pass): the
// largest chunks per lane a pass uses, waves per workgroup and rows per wave
// per batch, and which kernel: the shared-activation kernel (one format,
// one token row; batch = u rows of one wave), the matrix-core verify kernel
// (int4, 3..8 token rows; batch = u rows in 16-row tiles) or the register
// kernel (int4, two token rows; batch = u rows per row group).
// Device pointers of a prepared plan's workspace.
struct StepLaunch {
  const GemvArgs* mats;
  const int64_t* begin;   // range starts (groups + 1), cut on the host
  const int32_t* first;   // first matrix of each range
  StepCuts cuts;          // cost prefix and XCD balance (shared-activation kernel)
};

struct StepVariant {
  int cpl_max;
  int waves;
  int u;
  const void* kernel;
  void (*launch)(int grid, const StepLaunch&, hipStream_t);
  int cmax;    // > 0: the shared-activation kernel, staging at most cmax chunks of a row
  bool verify; // the matrix-core verify kernel
};

template <class F, int M, int CPL, int U, int WAVES, bool PF>
static void step_launch(int grid, const StepLaunch& l, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_step_kernel<F, M, CPL, U, WAVES, PF>), dim3((unsigned)grid), dim3(WAVES * 64), 0,
                     stream, l.mats, l.begin, l.first);
}

template <class F, int M, int CPL, int U, int WAVES, bool PF>
static StepVariant variant() {
  return StepVariant{CPL, WAVES, U, reinterpret_cast<const void*>(gemv_step_kernel<F, M, CPL, U, WAVES, PF>),
                     &step_launch<F, M, CPL, U, WAVES, PF>, 0, false};
}

template <class F, int U, int CPL, int WAVES, bool PF>
static void shared_launch(int grid, const StepLaunch& l, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_step_shared_kernel<F, U, CPL, WAVES, PF>), dim3((unsigned)grid), dim3(WAVES * 64), 0,
                     stream, l.mats, l.cuts);
}

template <class F, int U, int CPL, int WAVES, bool PF>
static StepVariant shared_variant() {
  return StepVariant{CPL, WAVES, U, reinterpret_cast<const void*>(gemv_step_shared_kernel<F, U, CPL, WAVES, PF>),
                     &shared_launch<F, U, CPL, WAVES, PF>, shared_x_cmax<F, CPL>(), false};
}

constexpr int kVerifyKW = 256, kVerifyRT = 2, kVerifyOct = 2;

template <int M, int WAVES, bool PF, int RT, int OCT, int KW, bool QL, bool SB>
static void verify_launch(int grid, const StepLaunch& l, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_verify_step_kernel<M, KW, WAVES, RT, OCT, PF, QL, SB>), dim3((unsigned)grid),
                     dim3(WAVES * 64), 0, stream, l.mats, l.begin, l.first);
}

template <int M, int WAVES, bool PF, int RT = kVerifyRT, int OCT = kVerifyOct, int KW = kVerifyKW, bool QL = true,
          bool SB = false>
static StepVariant verify_variant() {
  return StepVariant{1, WAVES, 16 * RT,
                     reinterpret_cast<const void*>(gemm_verify_step_kernel<M, KW, WAVES, RT, OCT, PF, QL, SB>),
                     &verify_launch<M, WAVES, PF, RT, OCT, KW, QL, SB>, 0, true};
}

static bool pick_variant(int format, int m, StepVariant& v) {
  // chosen by timing candidates on the Llama-2-7B / Llama-3.1-8B / -70B sets
  if (format == WQ_FORMAT_BF16 && m == 1) {
    v = shared_variant<FmtBf16, 4, 2, 16, true>();
  } else if (format == WQ_FORMAT_INT8 && m == 1) {
    v = shared_variant<FmtInt8, 2, 2, 16, true>();
  } else if (format == WQ_FORMAT_INT4G32) {
    switch (m) {
      case 1: v = shared_variant<FmtInt4, 2, 2, 16, true>(); break;
      case 2: v = variant<FmtInt4, 2, 2, 2, 8, false>(); break;
      case 3: v = verify_variant<3, 12, true>(); break;
      case 4: v = verify_variant<4, 12, true>(); break;
      case 5: v = verify_variant<5, 8, true>(); break;
      case 6: v = verify_variant<6, 8, true, 2, 2, 128>(); break;
      case 7: v = verify_variant<7, 8, true, 2, 2, 128>(); break;
      case 8: v = verify_variant<8, 8, true, 2, 2, 128>(); break;
      default: return false;
    }
  } else {
    return false;
  }
  return true;
}

static int weights_per_chunk(int format) {
  return format == WQ_FORMAT_BF16 ? 8 : (format == WQ_FORMAT_INT8 ? 16 : 32);
}

static int64_t row_bytes_of(int format, int64_t k) {
  return format == WQ_FORMAT_BF16 ? 2 * k : (format == WQ_FORMAT_INT8 ? k : k / 2);
}

constexpr int kMaxGroups = 8192;   // workgroups of one step launch (upper bound)

// Workspace layout: per-matrix descriptors, the range starts of the
// workgroups (groups + 1) and the first matrix of each range (groups), the
// step's cost before each matrix (count + 1) and per batch of each matrix
// (count), then the XCD balance state.
struct StepLayout {
  size_t begin, first, prefix, bcost, bal, end;
};

static StepLayout step_layout(int64_t count, int64_t groups) {
  auto up16 = [](size_t v) { return (v + 15) / 16 * 16; };
  StepLayout l;
  l.begin = up16((size_t)count * sizeof(GemvArgs));
  l.first = l.begin + ((size_t)groups + 1) * 8;
  l.prefix = up16(l.first + (size_t)groups * 4);
  l.bcost = l.prefix + ((size_t)count + 1) * 8;
  l.bal = up16(l.bcost + (size_t)count * 8);
  l.end = l.bal + sizeof(StepBalance);
  return l;
}

static int64_t workspace_need(int64_t count, int64_t groups) { return (int64_t)step_layout(count, groups).end; }

static StepLaunch launch_view(void* workspace, int32_t count, int32_t groups, int64_t total) {
  char* ws = reinterpret_cast<char*>(workspace);
  const StepLayout l = step_layout(count, groups);
  StepLaunch v;
  v.mats = reinterpret_cast<const GemvArgs*>(ws);
  v.begin = reinterpret_cast<const int64_t*>(ws + l.begin);
  v.first = reinterpret_cast<const int32_t*>(ws + l.first);
  v.cuts.prefix = reinterpret_cast<const double*>(ws + l.prefix);
  v.cuts.bcost = reinterpret_cast<const double*>(ws + l.bcost);
  v.cuts.bal = reinterpret_cast<StepBalance*>(ws + l.bal);
  v.cuts.total = total;
  v.cuts.count = count;
  return v;
}

}  // namespace wq

using namespace wq;

extern "C" int64_t wq_decode_step_workspace_bytes(int32_t count) {
  if (count < 0) return 0;
  return workspace_need(count, kMaxGroups);
}

extern "C" int wq_decode_step_prepare(int32_t format, int32_t m, const wq_matrix* mats, int32_t count,
                                      void* workspace, int64_t workspace_bytes, wq_step_plan* plan) {
  const char* name = "wq_decode_step_prepare";
  if (!mats || !workspace || !plan) return fail(WQ_ERR_NULL, "%s: mats, workspace and plan must be non-null", name);
  if (count < 1) return fail(WQ_ERR_SHAPE, "%s: count = %d must be >= 1", name, count);
  StepVariant v{};
  if (!pick_variant(format, m, v))
    return fail(WQ_ERR_SHAPE, "%s: unsupported format %d with m = %d (m = 1 for bf16/int8, 1..8 for int4)", name,
                format, m);
  const int wpc = weights_per_chunk(format);
  std::vector<GemvArgs> desc((size_t)count);
  std::vector<double> batch_bytes((size_t)count);
  int64_t total_batches = 0;
  for (int32_t i = 0; i < count; ++i) {
    const wq_matrix& mt = mats[i];
    if (!mt.x || !mt.w || (format != WQ_FORMAT_BF16 && !mt.aux))
      return fail(WQ_ERR_NULL, "%s: matrix %d: x, w (and scales) must be non-null", name, i);
    if (!mt.y_f32 && !mt.y_bf16)
      return fail(WQ_ERR_NULL, "%s: matrix %d: at least one of y_f32 / y_bf16 must be non-null", name, i);
    if (mt.n < 1 || mt.k < wpc || mt.k % wpc || mt.n > ((int64_t)1 << 31))
      return fail(WQ_ERR_SHAPE, "%s: matrix %d: n = %lld, k = %lld (need n >= 1, k a positive multiple of %d)",
                  name, i, (long long)mt.n, (long long)mt.k, wpc);
    const int64_t chunks = mt.k / wpc;
    const int64_t per_wave_max = (int64_t)kWave * v.cpl_max;
    const int64_t split = v.cmax || v.verify ? 1 : (chunks + per_wave_max - 1) / per_wave_max;
    const int64_t passes = (chunks + per_wave_max - 1) / per_wave_max;
    if (split > v.waves || (v.verify && mt.k > kVerifyMaxK) || (v.cmax && passes * per_wave_max > v.cmax))
      return fail(WQ_ERR_SHAPE, "%s: matrix %d: k = %lld is larger than this step kernel supports", name, i,
                  (long long)mt.k);
    if (!aligned16(mt.x) || !aligned16(mt.w) ||
        (format == WQ_FORMAT_INT4G32 && (reinterpret_cast<uintptr_t>(mt.aux) & 3u)))
      return fail(WQ_ERR_ALIGN, "%s: matrix %d: x and w must be 16-byte aligned (sz 4-byte)", name, i);
    GemvArgs& a = desc[(size_t)i];
    a = GemvArgs{};
    a.x = reinterpret_cast<const uint16_t*>(mt.x);
    a.w = reinterpret_cast<const uint8_t*>(mt.w);
    if (format == WQ_FORMAT_INT8) a.scale = reinterpret_cast<const uint16_t*>(mt.aux);
    if (format == WQ_FORMAT_INT4G32) a.sz = reinterpret_cast<const uint32_t*>(mt.aux);
    a.y32 = mt.y_f32;
    a.y16 = mt.y_bf16;
    a.n = mt.n;
    a.k = mt.k;
    a.row_bytes = row_bytes_of(format, mt.k);
    a.chunks = (int32_t)chunks;
    a.split = (int32_t)split;
    a.groups = v.cmax || v.verify ? 1 : v.waves / (int32_t)split;
    // the shared-activation kernel streams a row in `passes` passes of cpl_max
    // chunks per lane
    a.cpl = v.cmax ? (int32_t)passes : (int32_t)((chunks + split * kWave - 1) / (split * kWave));
    // the verify kernel's batch is a block of 16-row tiles, the
    // shared-activation kernel's u rows of one wave
    const int64_t rows_per_batch = v.cmax || v.verify ? (int64_t)v.u : (int64_t)a.groups * v.u;
    a.batches = (a.n + rows_per_batch - 1) / rows_per_batch;
    a.batch_begin = total_batches;
    total_batches += a.batches;
    const double aux_bytes = format == WQ_FORMAT_INT4G32 ? (double)chunks * 4 : (format == WQ_FORMAT_INT8 ? 2 : 0);
    batch_bytes[(size_t)i] = (double)rows_per_batch * ((double)a.row_bytes + aux_bytes);
    // the shared-activation kernel spends arithmetic on every lane of a pass,
    // including the lanes past a row's end in its last pass: weigh a batch by
    // its padded length so that rows whose length is not a multiple of a
    // pass (e.g. k = 11008) get proportionally shorter ranges
    if (v.cmax) batch_bytes[(size_t)i] *= (double)(passes * per_wave_max) / (double)chunks;
  }
  int rc = check_device();
  if (rc) return rc;

  int groups = resident_groups(v.kernel, v.waves * kWave);
  if (groups > kMaxGroups) groups = kMaxGroups;
  if (groups > total_batches) groups = (int)total_batches;
  if (groups < 1) groups = 1;
  const int64_t need = workspace_need(count, groups);
  if (workspace_bytes < need)
    return fail(WQ_ERR_SHAPE, "%s: workspace of %lld bytes is smaller than the %lld needed", name,
                (long long)workspace_bytes, (long long)need);
  if (!aligned16(workspace)) return fail(WQ_ERR_ALIGN, "%s: workspace must be 16-byte aligned", name);

  // The first global batch at or after byte offset `target` of the step
  // (a batch belongs to the range its first byte falls in).
  double total = 0;
  for (int32_t i = 0; i < count; ++i) total += batch_bytes[(size_t)i] * (double)desc[(size_t)i].batches;
  auto batch_at = [&](double target) -> int64_t {
    double acc = 0;   // bytes before matrix i
    for (int32_t i = 0; i < count; ++i) {
      const double mb = batch_bytes[(size_t)i] * (double)desc[(size_t)i].batches;
      if (acc + mb > target) {
        int64_t local = (int64_t)((target - acc) / batch_bytes[(size_t)i] + 0.999999);
        if (local > desc[(size_t)i].batches) local = desc[(size_t)i].batches;
        return desc[(size_t)i].batch_begin + local;
      }
      acc += mb;
    }
    return total_batches;
  };
  auto matrix_of = [&](int64_t gb) -> int32_t {
    if (gb >= total_batches) gb = total_batches - 1;
    int32_t lo = 0, hi = count - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) / 2;
      if (desc[(size_t)mid].batch_begin <= gb) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };

  // [0, total_batches) cut into `groups` ranges of equal cost
  std::vector<int64_t> begin((size_t)groups + 1);
  std::vector<int32_t> first((size_t)groups);
  for (int g = 0; g <= groups; ++g) {
    int64_t gb = g == groups ? total_batches : batch_at(total * (double)g / (double)groups);
    if (gb > total_batches) gb = total_batches;
    if (g > 0 && gb < begin[(size_t)g - 1]) gb = begin[(size_t)g - 1];
    begin[(size_t)g] = gb;
  }
  for (int g = 0; g < groups; ++g) first[(size_t)g] = matrix_of(begin[(size_t)g]);

  const StepLayout lay = step_layout(count, groups);
  std::vector<char> host(lay.end, 0);
  memcpy(host.data(), desc.data(), (size_t)count * sizeof(GemvArgs));
  memcpy(host.data() + lay.begin, begin.data(), ((size_t)groups + 1) * 8);
  memcpy(host.data() + lay.first, first.data(), (size_t)groups * 4);
  std::vector<double> prefix((size_t)count + 1, 0.0);
  for (int32_t i = 0; i < count; ++i)
    prefix[(size_t)i + 1] = prefix[(size_t)i] + batch_bytes[(size_t)i] * (double)desc[(size_t)i].batches;
  memcpy(host.data() + lay.prefix, prefix.data(), prefix.size() * 8);
  memcpy(host.data() + lay.bcost, batch_bytes.data(), (size_t)count * 8);
  StepBalance bal{};
  for (int x = 0; x < 8; ++x) bal.w[x] = 1.0f;
  memcpy(host.data() + lay.bal, &bal, sizeof(bal));
  hipError_t e = hipMemcpy(workspace, host.data(), host.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(WQ_ERR_LAUNCH, "%s: copying the plan to the workspace failed: %s", name, hipGetErrorString(e));
  }
  memset(plan, 0, sizeof(*plan));
  plan->format = format;
  plan->m = m;
  plan->count = count;
  plan->groups = groups;
  plan->workspace = workspace;
  plan->total_batches = total_batches;
  return WQ_OK;
}

extern "C" int wq_decode_step_run(const wq_step_plan* plan, void* stream) {
  const char* name = "wq_decode_step_run";
  if (!plan || !plan->workspace) return fail(WQ_ERR_NULL, "%s: plan and its workspace must be non-null", name);
  StepVariant v{};
  if (!pick_variant(plan->format, plan->m, v) || plan->count < 1 || plan->groups < 1 || plan->groups > kMaxGroups)
    return fail(WQ_ERR_SHAPE, "%s: the plan was not produced by wq_decode_step_prepare", name);
  int rc = check_device();
  if (rc) return rc;
  const StepLaunch l = launch_view(const_cast<void*>(plan->workspace), plan->count, plan->groups, plan->total_batches);
  v.launch(plan->groups, l, (hipStream_t)stream);
  return launch_status(name);
}
