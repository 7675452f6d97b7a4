// Whole decode step in one launch: plan once on the host, then launch the
// persistent step kernel (wq_step_shared.hpp for one token row, wq_verify.hpp
// for 2..8 with int4 G=32 weights, wq_step_i8mt.hpp for 2..8 with int8
// weights) as often as needed.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "wq_gemv_kernel.hpp"
#include "wq_host.hpp"
#include "wq_step_i8mt.hpp"
#include "wq_step_shared.hpp"
#include "wq_verify.hpp"

namespace wq {

// Device pointers of a prepared plan's workspace.
struct StepLaunch {
  const GemvArgs* mats;
  StepCuts cuts;          // cost prefix and per-workgroup balance (every step kernel)
  VerifyCuts vcuts;       // cost prefixes and long-row balance (verify kernel)
};

// One persistent kernel configuration per (format, tokens per pass): the
// largest chunks per lane a pass uses, waves per workgroup and rows per
// batch, and which kernel: the shared-activation kernel (one format, one
// token row; batch = u rows of one wave), the matrix-core verify kernel
// (int4, 2..8 token rows; batch = u rows in 16-row tiles) or the int8
// matrix-core kernel (2..8 token rows; batch = u rows in 16-row tiles that
// one wave streams, cpl_max chunks of each row per pass).
struct StepVariant {
  int cpl_max;
  int waves;
  int u;
  const void* kernel;
  void (*launch)(int grid, const StepLaunch&, hipStream_t);
  int cmax;    // > 0: the shared-activation kernel, staging at most cmax chunks of a row
  bool verify; // the matrix-core verify kernel
  int kw = 0;   // verify: groups of one staged activation window
  bool tiled = false;   // the int8 matrix-core kernel
};

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

template <int M, int U, int WAVES>
static void i8mt_launch(int grid, const StepLaunch& l, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_i8_step_kernel<M, U, WAVES>), dim3((unsigned)grid), dim3(WAVES * 64), 0, stream,
                     l.mats, l.cuts);
}

// 4 tiles (64 rows) per batch share each activation load; 8 waves
template <int M, int U = 4, int WAVES = 8>
static StepVariant i8mt_variant() {
  StepVariant v{kMtPassChunks, WAVES, 16 * U, reinterpret_cast<const void*>(gemm_i8_step_kernel<M, U, WAVES>),
                &i8mt_launch<M, U, WAVES>, 0, false};
  v.tiled = true;
  return v;
}

// the int8 matrix-core kernel addresses a matrix's codes and its M x k
// activations with 32-bit offsets below 0xFFFFFFE0 (larger ones mean "past
// the end")
constexpr int64_t kTiledMaxK = (int64_t)1 << 24;
constexpr int64_t kTiledMaxBytes = (int64_t)0xFFFFFF00u;

// starting value of the verify kernel's long-row cost factor (measured on
// the Llama-3.1-70B set: rows of 28672 inputs cost ~1.2x per byte); each
// launch refines it
constexpr double kVerifyLongRowPrior = 1.2;

template <int M, int WAVES, int RT, int OCT, int KW, bool LT>
static void verify_launch(int grid, const StepLaunch& l, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_verify_step_kernel<M, KW, WAVES, RT, OCT, LT>), dim3((unsigned)grid),
                     dim3(WAVES * 64), 0, stream, l.mats, l.vcuts);
}

// LT: codes loaded line-wide and moved to the MFMA layout through a per-wave
// LDS tile (2 KiB per wave on top of the activation window), else quad-row
// loads and cross-lane permutes.
template <int M, int WAVES, int RT, int OCT, int KW, bool LT>
static StepVariant verify_variant() {
  return StepVariant{1, WAVES, 16 * RT,
                     reinterpret_cast<const void*>(gemm_verify_step_kernel<M, KW, WAVES, RT, OCT, LT>),
                     &verify_launch<M, WAVES, RT, OCT, KW, LT>, 0, true, KW};
}

template <int M>
static StepVariant verify_config_variant() {
  using C = VerifyConfig<M>;
  return verify_variant<M, C::kWaves, C::kRT, C::kOct, C::kKW, C::kLT>();
}

static bool is_int4(int format) {
  return (format >= WQ_FORMAT_INT4G32 && format <= WQ_FORMAT_INT4G256) || format == WQ_FORMAT_INT4PC;
}

static bool pick_variant(int format, int m, StepVariant& v) {
  // chosen by timing candidates on the Llama-2-7B / Llama-3.1-8B / -70B sets
  if (format == WQ_FORMAT_BF16 && m == 1) {
    v = shared_variant<FmtBf16, 4, 2, 16, true>();
  } else if (format == WQ_FORMAT_INT8 && m == 1) {
    v = shared_variant<FmtInt8, 2, 2, 16, true>();
  } else if (format == WQ_FORMAT_INT8) {
    switch (m) {
      case 2: v = i8mt_variant<2>(); break;
      case 3: v = i8mt_variant<3>(); break;
      case 4: v = i8mt_variant<4>(); break;
      case 5: v = i8mt_variant<5>(); break;
      case 6: v = i8mt_variant<6>(); break;
      case 7: v = i8mt_variant<7>(); break;
      case 8: v = i8mt_variant<8>(); break;
      default: return false;
    }
  } else if (is_int4(format)) {
    // every group size (up to one group per row) runs the same kernels, each
    // 32-input chunk reading its group's (scale, zero) word
    switch (m) {
      case 1: v = shared_variant<FmtInt4, 2, 2, 16, true>(); break;
      case 2: v = verify_config_variant<2>(); break;
      case 3: v = verify_config_variant<3>(); break;
      case 4: v = verify_config_variant<4>(); break;
      case 5: v = verify_config_variant<5>(); break;
      case 6: v = verify_config_variant<6>(); break;
      case 7: v = verify_config_variant<7>(); break;
      case 8: v = verify_config_variant<8>(); break;
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

// int4: log2(group / 32), or kPerRowShift for one group per row
static int int4_gshift(int format) {
  if (format == WQ_FORMAT_INT4PC) return kPerRowShift;
  return is_int4(format) ? format - WQ_FORMAT_INT4G32 : 0;
}

static int64_t row_bytes_of(int format, int64_t k) {
  return format == WQ_FORMAT_BF16 ? 2 * k : (format == WQ_FORMAT_INT8 ? k : k / 2);
}

constexpr int kMaxGroups = kStepMaxGroups;   // workgroups of one step launch (upper bound)

// Workspace layout: per-matrix descriptors, the step's cost before each
// matrix (count + 1; for the verify kernel: of the short-row matrices), the
// long-row cost before each matrix (count + 1, verify kernel), the cost per
// batch of each matrix (count), then the per-workgroup balance state and the
// verify kernel's long-row balance state.  Workgroups cut their ranges from these
// on the device.
struct StepLayout {
  size_t prefix, prefl, bcost, bal, vbal, end;
};

static StepLayout step_layout(int64_t count) {
  auto up16 = [](size_t v) { return (v + 15) / 16 * 16; };
  StepLayout l;
  l.prefix = up16((size_t)count * sizeof(GemvArgs));
  l.prefl = l.prefix + ((size_t)count + 1) * 8;
  l.bcost = l.prefl + ((size_t)count + 1) * 8;
  l.bal = up16(l.bcost + (size_t)count * 8);
  l.vbal = up16(l.bal + sizeof(StepBalance));
  l.end = l.vbal + sizeof(VerifyBalance);
  return l;
}

static int64_t workspace_need(int64_t count) { return (int64_t)step_layout(count).end; }

static StepLaunch launch_view(void* workspace, int32_t count, int64_t total) {
  char* ws = reinterpret_cast<char*>(workspace);
  const StepLayout l = step_layout(count);
  StepLaunch v;
  v.mats = reinterpret_cast<const GemvArgs*>(ws);
  v.cuts.prefix = reinterpret_cast<const double*>(ws + l.prefix);
  v.cuts.bcost = reinterpret_cast<const double*>(ws + l.bcost);
  v.cuts.bal = reinterpret_cast<StepBalance*>(ws + l.bal);
  v.cuts.total = total;
  v.cuts.count = count;
  v.vcuts.pre_short = v.cuts.prefix;
  v.vcuts.pre_long = reinterpret_cast<const double*>(ws + l.prefl);
  v.vcuts.bcost = v.cuts.bcost;
  v.vcuts.bal = reinterpret_cast<VerifyBalance*>(ws + l.vbal);
  v.vcuts.wg = v.cuts.bal;
  v.vcuts.count = count;
  return v;
}

}  // namespace wq

using namespace wq;

extern "C" int64_t wq_decode_step_workspace_bytes(int32_t count) {
  if (count < 0) return 0;
  return workspace_need(count);
}

extern "C" int wq_decode_step_prepare(int32_t format, int32_t m, const wq_matrix* mats, int32_t count,
                                      void* workspace, int64_t workspace_bytes, wq_step_plan* plan) {
  const char* name = "wq_decode_step_prepare";
  if (!mats || !workspace || !plan) return fail(WQ_ERR_NULL, "%s: mats, workspace and plan must be non-null", name);
  if (count < 1) return fail(WQ_ERR_SHAPE, "%s: count = %d must be >= 1", name, count);
  StepVariant v{};
  if (!pick_variant(format, m, v))
    return fail(WQ_ERR_SHAPE, "%s: unsupported format %d with m = %d (m = 1 for bf16, 1..8 for int8 and int4)", name,
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
    // int4 with groups of G: k a multiple of G; one group per row: of 32
    const int kmult = format == WQ_FORMAT_INT4PC ? wpc : wpc << int4_gshift(format);
    if (mt.n < 1 || mt.k < kmult || mt.k % kmult || mt.n > ((int64_t)1 << 31))
      return fail(WQ_ERR_SHAPE, "%s: matrix %d: n = %lld, k = %lld (need n >= 1, k a positive multiple of %d)",
                  name, i, (long long)mt.n, (long long)mt.k, kmult);
    const int64_t chunks = mt.k / wpc;
    // chunks of a row one pass covers
    const int64_t per_wave_max = v.tiled ? (int64_t)v.cpl_max : (int64_t)kWave * v.cpl_max;
    const int64_t passes = (chunks + per_wave_max - 1) / per_wave_max;
    if ((v.verify && mt.k > kVerifyMaxK) || (v.cmax && passes * per_wave_max > v.cmax) ||
        (v.tiled && (mt.k > kTiledMaxK || mt.n * row_bytes_of(format, mt.k) > kTiledMaxBytes)))
      return fail(WQ_ERR_SHAPE, "%s: matrix %d: k = %lld is larger than this step kernel supports", name, i,
                  (long long)mt.k);
    if (!aligned16(mt.x) || !aligned16(mt.w) ||
        (is_int4(format) && (reinterpret_cast<uintptr_t>(mt.aux) & 3u)))
      return fail(WQ_ERR_ALIGN, "%s: matrix %d: x and w must be 16-byte aligned (sz 4-byte)", name, i);
    GemvArgs& a = desc[(size_t)i];
    a = GemvArgs{};
    a.x = reinterpret_cast<const uint16_t*>(mt.x);
    a.w = reinterpret_cast<const uint8_t*>(mt.w);
    if (format == WQ_FORMAT_INT8) a.scale = reinterpret_cast<const uint16_t*>(mt.aux);
    if (is_int4(format)) a.sz = reinterpret_cast<const uint32_t*>(mt.aux);
    a.gshift = int4_gshift(format);
    a.y32 = mt.y_f32;
    a.y16 = mt.y_bf16;
    a.n = mt.n;
    a.k = mt.k;
    a.row_bytes = row_bytes_of(format, mt.k);
    a.chunks = (int32_t)chunks;
    a.split = 1;
    a.groups = 1;
    // the shared-activation and int8 matrix-core kernels stream a row in
    // `passes` passes
    a.cpl = (v.cmax || v.tiled) ? (int32_t)passes : 1;
    // one-token kernels: rows of one pass that would leave half the lanes
    // idle share a wave pass, L = 64 / rpp lanes each (L >= 8 and L * CPL
    // chunks cover the row).  A lane holds u x CPL chunk slots: CPL chunks of
    // each of u rows, or ("wide") up to u * CPL chunks of one row, whichever
    // leaves fewer slots past the row's end (a 43-chunk row: 32 lanes x 2
    // fill 67 % of the slots, 16 lanes x 3 fill 90 %)
    a.rpp = 1;
    a.wide = 0;
    int64_t slots = passes * per_wave_max;   // chunk slots a row costs (arithmetic)
    if (!v.tiled && !v.verify && passes == 1) {
      const int64_t lanes = (chunks + v.cpl_max - 1) / v.cpl_max;
      int L = kWave;
      while (L > 8 && L / 2 >= lanes) L /= 2;
      const int64_t s_pair = (int64_t)L * v.cpl_max;
      const int64_t per_lane = (int64_t)v.u * v.cpl_max;
      int Lw = kWave;
      while (Lw > 8 && (int64_t)(Lw / 2) * per_lane >= chunks) Lw /= 2;
      const int64_t s_wide = (int64_t)Lw * ((chunks + Lw - 1) / Lw);
      if (format != WQ_FORMAT_INT8 && Lw < kWave && 10 * s_pair >= 11 * s_wide) {
        // wide pays off when it uses at least ~10 % more of its slots (not
        // for int8, whose kernel has no wide passes)
        a.rpp = kWave / Lw;
        a.wide = 1;
        slots = s_wide;
      } else {
        a.rpp = kWave / L;
        if (a.rpp > 1) slots = s_pair;
      }
    }
    // the verify kernel's batch is a block of 16-row tiles, the
    // shared-activation kernel's u rows of one wave (u x rpp with short rows;
    // rpp rows when wide)
    const int64_t rows_per_batch = a.wide ? (int64_t)a.rpp : (int64_t)v.u * a.rpp;
    a.batches = (a.n + rows_per_batch - 1) / rows_per_batch;
    a.batch_begin = total_batches;
    total_batches += a.batches;
    const double aux_bytes =
        is_int4(format) ? (double)int4_row_words(chunks, a.gshift) * 4 : (format == WQ_FORMAT_INT8 ? 2 : 0);
    batch_bytes[(size_t)i] = (double)rows_per_batch * ((double)a.row_bytes + aux_bytes);
    // the streaming kernels spend arithmetic on every lane of a pass,
    // including the lanes past a row's end in its last pass: weigh a batch by
    // its padded length so that rows whose length is not a multiple of a
    // pass (e.g. k = 11008) get proportionally shorter ranges
    if (v.cmax || v.tiled) batch_bytes[(size_t)i] *= (double)(v.tiled ? passes * per_wave_max : slots) / (double)chunks;
  }
  int rc = check_device();
  if (rc) return rc;

  int groups = resident_groups(v.kernel, v.waves * kWave);
  if (groups > kMaxGroups) groups = kMaxGroups;
  if (groups > total_batches) groups = (int)total_batches;
  if (groups < 1) groups = 1;
  const int64_t need = workspace_need(count);
  if (workspace_bytes < need)
    return fail(WQ_ERR_SHAPE, "%s: workspace of %lld bytes is smaller than the %lld needed", name,
                (long long)workspace_bytes, (long long)need);
  if (!aligned16(workspace)) return fail(WQ_ERR_ALIGN, "%s: workspace must be 16-byte aligned", name);

  const StepLayout lay = step_layout(count);
  std::vector<char> host(lay.end, 0);
  memcpy(host.data(), desc.data(), (size_t)count * sizeof(GemvArgs));
  // verify kernel: short-row and long-row bytes kept apart (the kernel weighs
  // the long ones by its balance factor); other kernels: prefl stays zero
  std::vector<double> prefix((size_t)count + 1, 0.0), prefl((size_t)count + 1, 0.0);
  for (int32_t i = 0; i < count; ++i) {
    const double mb = batch_bytes[(size_t)i] * (double)desc[(size_t)i].batches;
    const bool is_long = v.verify && desc[(size_t)i].chunks > v.kw;
    prefix[(size_t)i + 1] = prefix[(size_t)i] + (is_long ? 0.0 : mb);
    prefl[(size_t)i + 1] = prefl[(size_t)i] + (is_long ? mb : 0.0);
  }
  memcpy(host.data() + lay.prefix, prefix.data(), prefix.size() * 8);
  memcpy(host.data() + lay.prefl, prefl.data(), prefl.size() * 8);
  memcpy(host.data() + lay.bcost, batch_bytes.data(), (size_t)count * 8);
  // equal shares to begin with: every workgroup weighs 1
  StepBalance* bal = reinterpret_cast<StepBalance*>(host.data() + lay.bal);
  for (int g = 0; g < groups; ++g) bal->w[g] = 1.0f;
  for (int p = 0; p < 2; ++p) {
    for (int g = 0; g < groups; ++g) bal->cum[p][g] = (double)g / (double)groups;
    bal->cum[p][groups] = 1.0;
  }
  VerifyBalance vbal{};
  vbal.f = kVerifyLongRowPrior;
  memcpy(host.data() + lay.vbal, &vbal, sizeof(vbal));
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
  const StepLaunch l = launch_view(const_cast<void*>(plan->workspace), plan->count, plan->total_batches);
  v.launch(plan->groups, l, (hipStream_t)stream);
  return launch_status(name);
}
