// Whole decode step in one launch: plan once on the host, then launch the
// persistent step kernel (wq_gemv_kernel.hpp) as often as needed.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "wq_gemv_kernel.hpp"
#include "wq_host.hpp"
#include "wq_mfma.hpp"
#include "wq_step_shared.hpp"
#include "wq_verify.hpp"

namespace wq {

// One persistent kernel configuration per (format, tokens per pass): the
// largest chunks-per-lane any matrix may use (registers are sized for it),
// waves per workgroup, rows per wave per batch and prefetch; or, for int4
// with 3..8 tokens, the matrix-core kernel (batch = one block of rows).
struct StepVariant {
  int cpl_max;
  int waves;
  int u;
  const void* kernel;
  void (*launch)(int grid, const void*, const int64_t*, const int32_t*, StepTail*, hipStream_t);
  bool mfma;   // int4 with 3..8 tokens: the matrix-core step kernel
  int cmax;    // > 0: the shared-activation kernel (batch = u rows of one wave),
               // staging at most cmax chunks of a row
  bool verify; // int4 with 2..8 tokens on the matrix cores, weights as the B
               // operand (batch = one 16-row tile)
  // dynamic tail (VALU kernel): fraction of the step's bytes handed out in
  // units of about `unit_bytes`; 0 = all static
  double tail_frac;
  double unit_bytes;
};

template <class F, int M, int CPL, int U, int WAVES, bool PF>
static void step_launch(int grid, const void* mats, const int64_t* begin, const int32_t* mat, StepTail* tail,
                        hipStream_t stream) {
  hipLaunchKernelGGL((gemv_step_kernel<F, M, CPL, U, WAVES, PF>), dim3((unsigned)grid), dim3(WAVES * 64), 0,
                     stream, reinterpret_cast<const GemvArgs*>(mats), begin, mat, tail);
}

template <class F, int M, int CPL, int U, int WAVES, bool PF>
static StepVariant variant() {
  return StepVariant{CPL, WAVES, U, reinterpret_cast<const void*>(gemv_step_kernel<F, M, CPL, U, WAVES, PF>),
                     &step_launch<F, M, CPL, U, WAVES, PF>, false, 0, false, 0.0, 0.0};
}

template <class F, int U, int CPL, int WAVES, bool PF>
static void shared_launch(int grid, const void* mats, const int64_t* begin, const int32_t* mat, StepTail*,
                          hipStream_t stream) {
  hipLaunchKernelGGL((gemv_step_shared_kernel<F, U, CPL, WAVES, PF>), dim3((unsigned)grid), dim3(WAVES * 64), 0,
                     stream, reinterpret_cast<const GemvArgs*>(mats), begin, mat);
}

template <class F, int U, int CPL, int WAVES, bool PF>
static StepVariant shared_variant() {
  return StepVariant{CPL, WAVES, U, reinterpret_cast<const void*>(gemv_step_shared_kernel<F, U, CPL, WAVES, PF>),
                     &shared_launch<F, U, CPL, WAVES, PF>, false, shared_x_cmax<F, CPL>(), false, 0.0, 0.0};
}

template <int M>
static void mfma_step_launch(int grid, const void* mats, const int64_t* begin, const int32_t* mat, StepTail*,
                             hipStream_t stream) {
  hipLaunchKernelGGL((gemm_mfma_step_kernel<M, kMfmaRT, kMfmaKW, kMfmaWaves, kMfmaPF, kMfmaOct>),
                     dim3((unsigned)grid), dim3(kMfmaWaves * 64), 0, stream, reinterpret_cast<const MfmaArgs*>(mats),
                     begin, mat);
}

template <int M>
static StepVariant mfma_variant() {
  return StepVariant{0, kMfmaWaves, 16 * kMfmaRT,
                     reinterpret_cast<const void*>(
                         gemm_mfma_step_kernel<M, kMfmaRT, kMfmaKW, kMfmaWaves, kMfmaPF, kMfmaOct>),
                     &mfma_step_launch<M>, true, 0, false, 0.0, 0.0};
}

constexpr int kVerifyKW = 256, kVerifyRT = 2, kVerifyOct = 2;

template <int M, int WAVES, bool PF, int RT, int OCT, int KW, bool QL>
static void verify_launch(int grid, const void* mats, const int64_t* begin, const int32_t* mat, StepTail*,
                          hipStream_t stream) {
  hipLaunchKernelGGL((gemm_verify_step_kernel<M, KW, WAVES, RT, OCT, PF, QL>), dim3((unsigned)grid),
                     dim3(WAVES * 64), 0, stream, reinterpret_cast<const GemvArgs*>(mats), begin, mat);
}

template <int M, int WAVES, bool PF, int RT = kVerifyRT, int OCT = kVerifyOct, int KW = kVerifyKW, bool QL = true>
static StepVariant verify_variant() {
  return StepVariant{1, WAVES, 16 * RT,
                     reinterpret_cast<const void*>(gemm_verify_step_kernel<M, KW, WAVES, RT, OCT, PF, QL>),
                     &verify_launch<M, WAVES, PF, RT, OCT, KW, QL>, false, 0, true, 0.0, 0.0};
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

// per-matrix descriptor slot: large enough for either kernel's descriptor
constexpr size_t kDescBytes = ((sizeof(GemvArgs) > sizeof(MfmaArgs) ? sizeof(GemvArgs) : sizeof(MfmaArgs)) + 15) / 16 * 16;

// Units of the dynamic tail (at most kMaxUnits per plan).
constexpr int64_t kMaxUnits = 65536;

// Workspace layout: descriptors, static range starts (groups + 1), first
// matrix per range (groups), then at a 16-byte boundary the tail header and
// the matrix of each tail unit.
static size_t tail_offset(size_t desc_bytes, int64_t count, int64_t groups) {
  const size_t off_first = (size_t)count * desc_bytes + ((size_t)groups + 1) * 8;
  return (off_first + (size_t)groups * 4 + 15) / 16 * 16;
}

static int64_t workspace_need(int64_t count, int64_t groups) {
  return (int64_t)tail_offset(kDescBytes, count, groups) + (int64_t)sizeof(StepTail) + 4 * kMaxUnits + 64;
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
    const int64_t per_wave_max = (int64_t)kWave * (v.mfma ? 1 : v.cpl_max);
    const int64_t split = v.mfma || v.cmax || v.verify ? 1 : (chunks + per_wave_max - 1) / per_wave_max;
    const int64_t passes = (chunks + per_wave_max - 1) / per_wave_max;
    if (split > v.waves || ((v.mfma || v.verify) && mt.k > kMfmaMaxK) || (v.cmax && passes * per_wave_max > v.cmax))
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
    // the matrix-core kernel's batch is one block of 16 * RT rows; the
    // shared-activation kernel's is u rows of one wave
    const int64_t rows_per_batch = v.mfma || v.cmax || v.verify ? (int64_t)v.u : (int64_t)a.groups * v.u;
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

  // Static part: [0, static_end) cut into `groups` equal-byte ranges; the
  // rest (for variants with a dynamic tail) is handed out in units.
  // Equal bytes take equal time only when the matrices share a shape; a
  // step that mixes row lengths streams them at different rates, so part of
  // it is handed out dynamically (variants with a tail only).
  bool mixed = false;
  for (int32_t i = 1; i < count; ++i) mixed = mixed || desc[(size_t)i].k != desc[0].k;
  const bool dynamic = !v.mfma && !v.cmax && !v.verify && groups > 1 && v.tail_frac > 0.0 && mixed;
  const double static_bytes = dynamic ? total * (1.0 - v.tail_frac) : total;
  const int64_t static_end = dynamic ? batch_at(static_bytes) : total_batches;
  std::vector<int64_t> begin((size_t)groups + 1);
  std::vector<int32_t> first((size_t)groups);
  for (int g = 0; g <= groups; ++g) {
    int64_t gb = g == groups ? static_end : batch_at(static_bytes * (double)g / (double)groups);
    if (gb > static_end) gb = static_end;
    if (g > 0 && gb < begin[(size_t)g - 1]) gb = begin[(size_t)g - 1];
    begin[(size_t)g] = gb;
  }
  for (int g = 0; g < groups; ++g) first[(size_t)g] = matrix_of(begin[(size_t)g]);

  StepTail tail{};
  std::vector<int32_t> unit_mat;
  if (dynamic && static_end < total_batches) {
    const int64_t left = total_batches - static_end;
    const double avg = (total - static_bytes) / (double)left;   // bytes per tail batch
    int64_t ub = (int64_t)(v.unit_bytes / avg + 0.5);
    if (ub < 1) ub = 1;
    if ((left + ub - 1) / ub > kMaxUnits) ub = (left + kMaxUnits - 1) / kMaxUnits;
    tail.units = (int32_t)((left + ub - 1) / ub);
    tail.start = static_end;
    tail.unit_batches = ub;
    tail.total = total_batches;
    unit_mat.resize((size_t)tail.units);
    for (int32_t u = 0; u < tail.units; ++u) unit_mat[(size_t)u] = matrix_of(static_end + (int64_t)u * ub);
  }

  char* ws = reinterpret_cast<char*>(workspace);
  const size_t desc_bytes = v.mfma ? sizeof(MfmaArgs) : sizeof(GemvArgs);
  const size_t off_begin = (size_t)count * desc_bytes;
  const size_t off_first = off_begin + ((size_t)groups + 1) * 8;
  const size_t off_tail = tail_offset(desc_bytes, count, groups);
  std::vector<char> host(off_tail + sizeof(StepTail) + unit_mat.size() * 4, 0);
  if (v.mfma) {
    std::vector<MfmaArgs> md((size_t)count);
    for (int32_t i = 0; i < count; ++i) {
      const GemvArgs& g = desc[(size_t)i];
      MfmaArgs& a = md[(size_t)i];
      a = MfmaArgs{};
      a.x = g.x;
      a.w = g.w;
      a.sz = g.sz;
      a.y32 = g.y32;
      a.y16 = g.y16;
      a.n = g.n;
      a.k = g.k;
      a.groups = (int32_t)(g.k / 32);
      a.blocks = g.batches;
      a.block_begin = g.batch_begin;
    }
    memcpy(host.data(), md.data(), off_begin);
  } else {
    memcpy(host.data(), desc.data(), off_begin);
  }
  memcpy(host.data() + off_begin, begin.data(), ((size_t)groups + 1) * 8);
  memcpy(host.data() + off_first, first.data(), (size_t)groups * 4);
  memcpy(host.data() + off_tail, &tail, sizeof(StepTail));
  if (!unit_mat.empty()) memcpy(host.data() + off_tail + sizeof(StepTail), unit_mat.data(), unit_mat.size() * 4);
  hipError_t e = hipMemcpy(ws, host.data(), host.size(), hipMemcpyHostToDevice);
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
  char* ws = reinterpret_cast<char*>(const_cast<void*>(plan->workspace));
  const size_t desc_bytes = v.mfma ? sizeof(MfmaArgs) : sizeof(GemvArgs);
  const size_t off_begin = (size_t)plan->count * desc_bytes;
  const size_t off_first = off_begin + ((size_t)plan->groups + 1) * 8;
  const size_t off_tail = tail_offset(desc_bytes, plan->count, plan->groups);
  v.launch(plan->groups, ws, reinterpret_cast<const int64_t*>(ws + off_begin),
           reinterpret_cast<const int32_t*>(ws + off_first), reinterpret_cast<StepTail*>(ws + off_tail),
           (hipStream_t)stream);
  return launch_status(name);
}
