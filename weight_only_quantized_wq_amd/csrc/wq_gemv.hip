// Batch-1 (and small-M) decode matvecs y = x . W^T over bf16, int8 per-row
// and int4 weights, streamed from HBM: launch planning and the C entry
// points.  The kernels are in wq_gemv_kernel.hpp (one token row; 2, 3 and 5
// rows on the vector ALU when WQ_SMALLM_ENGINE=valu asks for them),
// wq_mfma.hpp and wq_verify.hpp (2..8 int4 rows) and wq_step_i8mt.hpp (2..8
// int8 rows).
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "wq_gemv_kernel.hpp"
#include "wq_host.hpp"
#include "wq_mfma.hpp"
#include "wq_step_i8mt.hpp"
#include "wq_verify.hpp"

namespace wq {

// ---------------------------------------------------------------------------
// Host side: plan selection and launch.

using LaunchFn = int (*)(const GemvArgs&, int split, hipStream_t);

template <class F, int M, int CPL, int U, int WAVES, bool PF>
int launch_one(const GemvArgs& a0, int split, hipStream_t stream) {
  auto kern = gemv_kernel<F, M, CPL, U, WAVES, PF>;
  GemvArgs a = a0;
  a.split = split;
  a.groups = WAVES / split;
  const int threads = split * a.groups * kWave;
  const int resident = resident_groups(reinterpret_cast<const void*>(kern), threads);
  const int64_t rows_per_batch = (int64_t)a.groups * U;
  a.batches = (a.n + rows_per_batch - 1) / rows_per_batch;
  int64_t grid = balanced_grid(a.batches, resident);
  if (grid <= 0) return WQ_OK;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, stream, a);
  return launch_status("gemv");
}

// Launch plans.  A plan fixes the chunks of activations each lane holds
// (CPL), the waves per workgroup, the rows per wave per batch (U) and whether
// the next batch is prefetched (PF); the split (waves per row) follows from
// the row length.  Each format lists its plans in order with the largest row
// (in chunks) each should serve; the first that covers the row is used.  The
// table was chosen by timing every candidate on the Llama-2-7B,
// Llama-3.1-8B and Llama-3.1-70B linear shapes on MI355X.  A 4-wave
// workgroup may use up to 512 VGPRs per lane, an 8-wave one 256 and a
// 16-wave one 128; every plan fits its size without spilling.
struct PlanEntry {
  int max_chunks;
  int cpl;
  int waves;
  LaunchFn fn;
};

#define WQ_PLAN(MAXC, CPL, WAVES, U, PF) {MAXC, CPL, WAVES, &launch_one<F, M, CPL, U, WAVES, PF>}

template <class F, int M>
struct Plans;

template <>
struct Plans<FmtBf16, 1> {
  using F = FmtBf16;
  static constexpr int M = 1;
  static constexpr PlanEntry list[] = {WQ_PLAN(128, 2, 4, 2, true), WQ_PLAN(512, 8, 4, 1, true),
                                       WQ_PLAN(1792, 7, 4, 1, true), WQ_PLAN(4096, 8, 8, 1, true),
                                       WQ_PLAN(8192, 8, 16, 1, false)};
};
template <>
struct Plans<FmtInt8, 1> {
  using F = FmtInt8;
  static constexpr int M = 1;
  static constexpr PlanEntry list[] = {WQ_PLAN(64, 1, 4, 4, true), WQ_PLAN(256, 4, 4, 2, false),
                                       WQ_PLAN(896, 7, 4, 1, true), WQ_PLAN(3584, 7, 8, 1, true),
                                       WQ_PLAN(4096, 4, 16, 1, false)};
};
template <>
struct Plans<FmtInt4, 1> {
  using F = FmtInt4;
  static constexpr int M = 1;
  static constexpr PlanEntry list[] = {WQ_PLAN(128, 2, 4, 2, false), WQ_PLAN(384, 3, 4, 2, true),
                                       WQ_PLAN(896, 7, 4, 1, true), WQ_PLAN(3584, 7, 8, 1, true),
                                       WQ_PLAN(4096, 8, 8, 1, false)};
};
// Several token rows on the vector ALU: each token's activations stay in
// registers, one decode serves every token.  These plans are the measured
// alternative to the matrix-core kernels for 2, 3 and 5 rows (see
// use_valu for the routing and the timings behind it).
template <>
struct Plans<FmtInt4, 2> {
  using F = FmtInt4;
  static constexpr int M = 2;
  static constexpr PlanEntry list[] = {WQ_PLAN(1024, 2, 8, 2, false), WQ_PLAN(4096, 1, 16, 1, false)};
};
template <>
struct Plans<FmtInt4, 3> {
  using F = FmtInt4;
  static constexpr int M = 3;
  static constexpr PlanEntry list[] = {WQ_PLAN(512, 1, 8, 2, false), WQ_PLAN(4096, 1, 16, 1, false)};
};
template <>
struct Plans<FmtInt4, 5> {
  using F = FmtInt4;
  static constexpr int M = 5;
  static constexpr PlanEntry list[] = {WQ_PLAN(512, 1, 8, 1, false), WQ_PLAN(4096, 1, 16, 1, false)};
};
template <>
struct Plans<FmtInt8, 2> {
  using F = FmtInt8;
  static constexpr int M = 2;
  static constexpr PlanEntry list[] = {WQ_PLAN(1024, 2, 8, 1, false), WQ_PLAN(4096, 1, 16, 1, false)};
};
template <>
struct Plans<FmtInt8, 3> {
  using F = FmtInt8;
  static constexpr int M = 3;
  static constexpr PlanEntry list[] = {WQ_PLAN(512, 1, 8, 2, false), WQ_PLAN(4096, 1, 16, 1, false)};
};
template <>
struct Plans<FmtInt8, 5> {
  using F = FmtInt8;
  static constexpr int M = 5;
  static constexpr PlanEntry list[] = {WQ_PLAN(512, 1, 8, 1, false), WQ_PLAN(4096, 1, 16, 1, false)};
};
#undef WQ_PLAN

template <class F, int M>
bool choose_plan(int64_t chunks, PlanEntry& best, int& split) {
  for (const PlanEntry& p : Plans<F, M>::list) {
    if (chunks > p.max_chunks) continue;
    const int64_t per_wave = (int64_t)kWave * p.cpl;
    int64_t s = chunks == 0 ? 1 : (chunks + per_wave - 1) / per_wave;
    if (s > p.waves) continue;
    best = p;
    split = (int)s;
    return true;
  }
  return false;
}

template <class F, int M>
int run_gemv(GemvArgs a, hipStream_t stream, const char* name) {
  PlanEntry p{};
  int split = 0;
  if (!choose_plan<F, M>(a.chunks, p, split))
    return fail(WQ_ERR_SHAPE, "%s: k = %lld is larger than the largest supported row", name, (long long)a.k);
  return p.fn(a, split, stream);
}

// Host checks in a fixed order -- null pointers, then sizes, then alignment --
// so a call is rejected for the first problem in that order.  `aux` is the
// scale (int8) or scale/zero (int4) array, checked when `need_aux`.
// log2(group / 32) for the int4 group sizes 32..256; kPerRowShift for one
// group per row (group == k, k a positive multiple of 32, checked by the
// caller); -1 otherwise
static int int4_group_shift(int64_t group, int64_t k) {
  switch (group) {
    case 32: return 0;
    case 64: return 1;
    case 128: return 2;
    case 256: return 3;
    default: return (group == k && k > 0) ? kPerRowShift : -1;
  }
}

// `group` >= 0 (int4): the group size, checked with the sizes; -1: no groups.
// `max_bytes` > 0: a bound on the n x row_bytes weight bytes, checked with
// the sizes.
static int check_common(const char* name, const void* x, const void* w, const void* aux, bool need_aux, int64_t n,
                        int64_t k, const float* y32, const uint16_t* y16, int kmult, int64_t m = 1,
                        int64_t group = -1, int64_t row_bytes = 0, int64_t max_bytes = 0) {
  if (!x || !w) return fail(WQ_ERR_NULL, "%s: x and the weights must be non-null", name);
  if (need_aux && !aux) return fail(WQ_ERR_NULL, "%s: the scale array must be non-null", name);
  if (!y32 && !y16) return fail(WQ_ERR_NULL, "%s: at least one of y_f32 / y_bf16 must be non-null", name);
  if (n < 0 || k < 0) return fail(WQ_ERR_SHAPE, "%s: negative size (n = %lld, k = %lld)", name, (long long)n, (long long)k);
  if (k % kmult != 0) return fail(WQ_ERR_SHAPE, "%s: k = %lld is not a multiple of %d", name, (long long)k, kmult);
  if (m < 1 || m > 8) return fail(WQ_ERR_SHAPE, "%s: m = %lld outside [1, 8]", name, (long long)m);
  if (n > ((int64_t)1 << 31)) return fail(WQ_ERR_SHAPE, "%s: n = %lld too large", name, (long long)n);
  if (k > ((int64_t)1 << 24)) return fail(WQ_ERR_SHAPE, "%s: k = %lld too large", name, (long long)k);
  if (group >= 0 && int4_group_shift(group, k) < 0)
    return fail(WQ_ERR_SHAPE, "%s: group = %lld (need 32, 64, 128, 256 or k = %lld)", name, (long long)group,
                (long long)k);
  if (group > 0 && k % group)
    return fail(WQ_ERR_SHAPE, "%s: k = %lld is not a multiple of group %lld", name, (long long)k, (long long)group);
  if (max_bytes > 0 && n * row_bytes > max_bytes)
    return fail(WQ_ERR_SHAPE, "%s: %lld weight bytes (n = %lld, k = %lld) exceed %lld", name,
                (long long)(n * row_bytes), (long long)n, (long long)k, (long long)max_bytes);
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
                     int64_t k, float* y_f32, uint16_t* y_bf16, GemvArgs& a, int64_t m = 1, int64_t group = 32) {
  int rc = check_common(name, x, qpacked, sz, true, n, k, y_f32, y_bf16, 32, m, group);
  if (rc) return rc;
  const int gshift = int4_group_shift(group, k);
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
  a.gshift = gshift;
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

extern "C" int wq_gemv_int4(const uint16_t* x, const uint8_t* qpacked, const uint16_t* sz, int64_t n, int64_t k,
                            int32_t group, float* y_f32, uint16_t* y_bf16, void* stream) {
  GemvArgs a;
  int rc = int4_args("wq_gemv_int4", x, qpacked, sz, n, k, y_f32, y_bf16, a, 1, group);
  if (rc) return rc;
  if (n == 0) return WQ_OK;
  if ((rc = check_device())) return rc;
  return run_gemv<FmtInt4, 1>(a, (hipStream_t)stream, "wq_gemv_int4");
}

namespace wq {

// Verify product on the matrix cores (2 <= m <= 8): workgroups of 12 waves
// over blocks of RT 16-row tiles, activations staged in LDS 256 groups (8192
// inputs) at a time, work items of 8 groups, one item prefetched.
template <int M, int RT>
int launch_mfma_rt(const GemvArgs& g, hipStream_t stream) {
  constexpr int KW = kMfmaKW, WAVES = kMfmaWaves, PF = kMfmaPF, OCT = kMfmaOct;
  constexpr bool LT = M <= 7;   // the code tile fits beside the activation window
  auto kern = gemm_mfma_kernel<M, RT, KW, WAVES, PF, OCT, LT>;
  const int resident = resident_groups(reinterpret_cast<const void*>(kern), WAVES * kWave);
  MfmaArgs a{};
  a.x = g.x;
  a.w = g.w;
  a.sz = g.sz;
  a.y32 = g.y32;
  a.y16 = g.y16;
  a.n = g.n;
  a.k = g.k;
  a.groups = (int32_t)(g.k / 32);
  a.gshift = g.gshift;
  a.words = int4_row_words(a.groups, g.gshift);
  a.blocks = (g.n + 16 * RT - 1) / (16 * RT);
  const int64_t grid = balanced_grid(a.blocks, resident);
  if (grid <= 0) return WQ_OK;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WAVES * kWave), 0, stream, a);
  return launch_status("wq_gemm_smallM");
}

// Blocks of two tiles share each staged activation read between them, which
// made one-tile blocks up to 25 % slower per tile (32000 x 4096: 13 % with
// the same tiles per workgroup); one tile per block only where that gives a
// workgroup at least a quarter fewer tiles (the largest workgroup share sets
// the launch's time): 10240 x 8192 at 5 tokens 19.4 -> 18.0 us, 12288 x
// 4096 12.6 -> 11.9 us.
template <int M>
int launch_mfma(const GemvArgs& g, hipStream_t stream) {
  constexpr int kSlots = 256;   // one workgroup per CU
  const int64_t tiles = (g.n + 15) / 16;
  const int64_t per2 = 2 * (((tiles + 1) / 2 + kSlots - 1) / kSlots);   // tiles per workgroup, two-tile blocks
  const int64_t per1 = (tiles + kSlots - 1) / kSlots;                   // one-tile blocks
  if (4 * per1 <= 3 * per2) return launch_mfma_rt<M, 1>(g, stream);
  return launch_mfma_rt<M, kMfmaRT>(g, stream);
}

}  // namespace wq

namespace wq {

// Claim slots of the single-matrix verify kernel, one per launch in turn;
// each launch leaves its slot zero.  Up to kMatrixClaimSlots launches may be
// in flight on one device at once.
constexpr int kMatrixClaimSlots = 1024;
static __device__ MatrixClaim g_matrix_claims[kMatrixClaimSlots];

static MatrixClaim* matrix_claim_slot() {
  static std::atomic<MatrixClaim*> base[kMaxDevices];
  static std::atomic<uint32_t> seq{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  MatrixClaim* p = base[dev].load(std::memory_order_acquire);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(g_matrix_claims)) != hipSuccess || !q) return nullptr;
    p = static_cast<MatrixClaim*>(q);
    base[dev].store(p, std::memory_order_release);
  }
  return p + seq.fetch_add(1, std::memory_order_relaxed) % kMatrixClaimSlots;
}

// Verify product with the weights in the B operand (gemm_verify_matrix_kernel,
// rows within one activation window): 8 waves over blocks of 32 rows, the
// step kernel's per-token-count windows; blocks past each workgroup's first
// are claimed as the workgroups go.
template <int M>
int launch_verify_matrix(const GemvArgs& g, hipStream_t stream) {
  constexpr int RT = 2, WAVES = 8, OCT = M == 4 ? 2 : 4, KW = VerifyConfig<M>::kKW;
  auto kern = gemm_verify_matrix_kernel<M, KW, WAVES, RT, OCT, true>;
  const int resident = resident_groups(reinterpret_cast<const void*>(kern), WAVES * kWave);
  GemvArgs a = g;
  a.batches = (g.n + 16 * RT - 1) / (16 * RT);
  const int64_t grid = a.batches < resident ? a.batches : resident;
  if (grid <= 0) return WQ_OK;
  // every workgroup may take up to `cap` blocks; grid * (cap - 1) blocks past
  // the first ones must cover the matrix
  const int64_t per = (a.batches + grid - 1) / grid;
  if (per + 1 > kMatrixMaxLocal) return launch_mfma<M>(g, stream);
  const int32_t cap = (int32_t)(2 * per + 2 < kMatrixMaxLocal ? 2 * per + 2 : kMatrixMaxLocal);
  MatrixClaim* claim = matrix_claim_slot();
  if (!claim) return fail(WQ_ERR_LAUNCH, "wq_gemm_smallM: no claim slot on the current device");
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WAVES * kWave), 0, stream, a, claim, cap);
  return launch_status("wq_gemm_smallM");
}

// Which matrix-core kernel serves 2..5 int4 token rows of one matrix:
// gemm_mfma_kernel ("split": a workgroup's blocks in a fixed stride, each
// block's items dealt to its waves) or gemm_verify_matrix_kernel ("claim":
// (block, window) units claimed by the waves, blocks past the first two
// claimed by the workgroups).  "auto" takes claim where it was measured
// faster: rows that fill all eight waves' windows (k >= 8192, within one
// activation window) and at least 5 blocks per workgroup (57344 x 8192:
// 67.8 -> 59.8 us, 128256 x 8192: 131.8 -> 108.8 us at 5 tokens); on
// smaller or shorter matrices its staging and claims cost more than they
// save (32768 x 8192 even, 16384 x 8192 and k = 4096 up to 20 % slower).
// WQ_SMALLM_KERNEL=split or =claim forces one where it applies (read at each
// call), which is how the two are timed and tested against each other.
enum class VerifyKernel { kAuto, kSplit, kClaim };

static VerifyKernel smallm_kernel() {
  const char* v = getenv("WQ_SMALLM_KERNEL");
  if (v && strcmp(v, "split") == 0) return VerifyKernel::kSplit;
  if (v && strcmp(v, "claim") == 0) return VerifyKernel::kClaim;
  return VerifyKernel::kAuto;
}

static bool use_claim_kernel(int64_t m, int64_t n, int64_t chunks) {
  if (m < 2 || m > 5 || chunks <= 0) return false;
  if (chunks > (m == 2 ? VerifyConfig<2>::kKW : VerifyConfig<3>::kKW)) return false;
  const VerifyKernel kind = smallm_kernel();
  if (kind != VerifyKernel::kAuto) return kind == VerifyKernel::kClaim;
  const int64_t blocks = (n + 31) / 32;
  return chunks >= 8 * kSzWin && blocks >= 5 * 256;
}

}  // namespace wq

namespace wq {

// Which kernels serve 2..8 token rows: the matrix cores or, for the row
// counts that have vector-ALU plans (2, 3, 5), the vector ALU.  "auto" takes
// the measured choice per format and row count; the environment variable
// WQ_SMALLM_ENGINE=mfma or =valu forces one side where it exists (read at
// each call), which is how the two are timed and tested against each other.
enum class Engine { kAuto, kMfma, kValu };

static Engine smallm_engine() {
  const char* v = getenv("WQ_SMALLM_ENGINE");
  if (v && strcmp(v, "mfma") == 0) return Engine::kMfma;
  if (v && strcmp(v, "valu") == 0) return Engine::kValu;
  return Engine::kAuto;
}

// True when the vector-ALU plans of F serve m rows of `chunks` chunks.
template <class F, int M>
static bool valu_fits(int64_t chunks) {
  PlanEntry p{};
  int split = 0;
  return choose_plan<F, M>(chunks, p, split);
}

template <class F>
static bool valu_fits_m(int64_t m, int64_t chunks) {
  switch (m) {
    case 2: return valu_fits<F, 2>(chunks);
    case 3: return valu_fits<F, 3>(chunks);
    case 5: return valu_fits<F, 5>(chunks);
    default: return false;
  }
}

template <class F>
static int run_gemv_m(const GemvArgs& a, int64_t m, hipStream_t s, const char* name) {
  switch (m) {
    case 2: return run_gemv<F, 2>(a, s, name);
    case 3: return run_gemv<F, 3>(a, s, name);
    default: return run_gemv<F, 5>(a, s, name);
  }
}

// The measured routing (auto): the matrix cores for every row count.  Timed
// on the Llama-3.1-70B shapes (back-to-back single launches), they beat the
// vector-ALU plans at 2 rows (int4 on all five shapes by 3-14 %, int8 on
// four of five; only int8 10240 x 8192 was 10 % faster on the vector ALU)
// and by ~2x at 3 and 5 rows, where the vector ALU runs out of issue slots.
static bool use_valu(bool int8, int64_t m, int64_t chunks) {
  if (smallm_engine() != Engine::kValu) return false;
  return int8 ? valu_fits_m<FmtInt8>(m, chunks) : valu_fits_m<FmtInt4>(m, chunks);
}

}  // namespace wq

static int gemm_small_m_int4(const char* name, const uint16_t* x, int64_t m, const uint8_t* qpacked, const uint16_t* sz,
                             int64_t n, int64_t k, int64_t group, float* y_f32, uint16_t* y_bf16, void* stream) {
  GemvArgs a;
  int rc = int4_args(name, x, qpacked, sz, n, k, y_f32, y_bf16, a, m, group);
  if (rc) return rc;
  if (n == 0) return WQ_OK;
  if ((rc = check_device())) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (m == 1) return run_gemv<FmtInt4, 1>(a, s, name);
  if (k > kMfmaMaxK) return fail(WQ_ERR_SHAPE, "%s: k = %lld is larger than %d", name, (long long)k, kMfmaMaxK);
  if (use_valu(false, m, a.chunks)) return run_gemv_m<FmtInt4>(a, m, s, name);
  if (use_claim_kernel(m, n, a.chunks)) {
    switch (m) {
      case 2: return launch_verify_matrix<2>(a, s);
      case 3: return launch_verify_matrix<3>(a, s);
      case 4: return launch_verify_matrix<4>(a, s);
      default: return launch_verify_matrix<5>(a, s);
    }
  }
  switch (m) {
    case 2: return launch_mfma<2>(a, s);
    case 3: return launch_mfma<3>(a, s);
    case 4: return launch_mfma<4>(a, s);
    case 5: return launch_mfma<5>(a, s);
    case 6: return launch_mfma<6>(a, s);
    case 7: return launch_mfma<7>(a, s);
    default: return launch_mfma<8>(a, s);
  }
}

extern "C" int wq_gemm_smallM(const uint16_t* x, int64_t m, const uint8_t* qpacked, const uint16_t* sz, int64_t n,
                              int64_t k, float* y_f32, uint16_t* y_bf16, void* stream) {
  return gemm_small_m_int4("wq_gemm_smallM", x, m, qpacked, sz, n, k, 32, y_f32, y_bf16, stream);
}

extern "C" int wq_gemm_smallM_int4(const uint16_t* x, int64_t m, const uint8_t* qpacked, const uint16_t* sz, int64_t n,
                                   int64_t k, int32_t group, float* y_f32, uint16_t* y_bf16, void* stream) {
  return gemm_small_m_int4("wq_gemm_smallM_int4", x, m, qpacked, sz, n, k, group, y_f32, y_bf16, stream);
}

namespace wq {

// int8 with 2..8 token rows: 16-row tiles, passes of kMtPassChunks 16-input
// chunks per row, the passes split over kI8mWaves waves.
constexpr int kI8mWaves = 8;
constexpr int64_t kI8mMaxBytes = (int64_t)0xFFFFFF00u;   // codes addressed with 32-bit offsets

// U tiles per batch share each activation load.  Fewer tiles per batch
// keep more batches in the grid: 4 from kI8mWideRows rows on; 2 from
// kI8mMidRows rows on when the matrix holds at least kI8mMidBytes (rows
// long enough that one batch per CU streams for a while); else 1.
constexpr int64_t kI8mWideRows = 16384, kI8mMidRows = 8192, kI8mMidBytes = int64_t(1) << 27;

template <int M, int U>
int launch_i8m_u(GemvArgs a, hipStream_t stream) {
  auto kern = gemm_i8_smallm_kernel<M, U, kI8mWaves>;
  const int resident = resident_groups(reinterpret_cast<const void*>(kern), kI8mWaves * kWave);
  const int64_t chunks = a.k / 16, per_pass = kMtPassChunks;
  a.cpl = (int32_t)((chunks + per_pass - 1) / per_pass);
  a.batches = (a.n + 16 * U - 1) / (16 * U);
  const int64_t grid = balanced_grid(a.batches, resident);
  if (grid <= 0) return WQ_OK;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kI8mWaves * kWave), 0, stream, a);
  return launch_status("wq_gemm_smallM_int8");
}

template <int M>
int launch_i8m(const GemvArgs& a, hipStream_t stream) {
  if (a.n >= kI8mWideRows) return launch_i8m_u<M, 4>(a, stream);
  if (a.n >= kI8mMidRows && a.n * a.k >= kI8mMidBytes) return launch_i8m_u<M, 2>(a, stream);
  return launch_i8m_u<M, 1>(a, stream);
}

// The claiming int8 kernel (gemm_i8_matrix_kernel): batches of U tiles as
// above, units of kMtUnitPasses passes, batches past each workgroup's first
// two claimed as the workgroups go.
template <int M, int U>
int launch_i8m_claim_u(GemvArgs a, hipStream_t stream) {
  auto kern = gemm_i8_matrix_kernel<M, U, kI8mWaves>;
  const int resident = resident_groups(reinterpret_cast<const void*>(kern), kI8mWaves * kWave);
  const int64_t chunks = a.k / 16, per_pass = kMtPassChunks;
  a.cpl = (int32_t)((chunks + per_pass - 1) / per_pass);
  a.batches = (a.n + 16 * U - 1) / (16 * U);
  const int64_t grid = a.batches < resident ? a.batches : resident;
  if (grid <= 0) return WQ_OK;
  const int64_t per = (a.batches + grid - 1) / grid;
  if (per + 1 > kMatrixMaxLocal) return launch_i8m_u<M, U>(a, stream);
  const int32_t cap = (int32_t)(2 * per + 2 < kMatrixMaxLocal ? 2 * per + 2 : kMatrixMaxLocal);
  MatrixClaim* claim = matrix_claim_slot();
  if (!claim) return fail(WQ_ERR_LAUNCH, "wq_gemm_smallM_int8: no claim slot on the current device");
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kI8mWaves * kWave), 0, stream, a, claim, cap);
  return launch_status("wq_gemm_smallM_int8");
}

template <int M>
int launch_i8m_claim(const GemvArgs& a, hipStream_t stream) {
  if (a.n >= kI8mWideRows) return launch_i8m_claim_u<M, 4>(a, stream);
  if (a.n >= kI8mMidRows && a.n * a.k >= kI8mMidBytes) return launch_i8m_claim_u<M, 2>(a, stream);
  return launch_i8m_claim_u<M, 1>(a, stream);
}

// int8 counterpart of use_claim_kernel (rows of up to kMtMaxUnits units).
// The int8 kernels are held by their decode arithmetic more than by how
// the work is spread: at 2, 5 and 8 tokens the claiming kernel was measured
// 2-3 % faster on 128256 x 8192, even on 57344 x 8192, and 10-30 % slower on
// 28672 x 8192 and smaller or on 8192 x 28672, so "auto" takes it only from
// 98304 rows on.
static bool use_claim_kernel_i8(int64_t n, int64_t k) {
  if (k <= 0 || k > (int64_t)kMtMaxUnits * kMtUnitPasses * 16 * kMtPassChunks) return false;
  const VerifyKernel kind = smallm_kernel();
  if (kind != VerifyKernel::kAuto) return kind == VerifyKernel::kClaim;
  return k >= 8192 && n >= 98304;
}

}  // namespace wq

extern "C" int wq_gemm_smallM_int8(const uint16_t* x, int64_t m, const int8_t* q, const uint16_t* scale, int64_t n,
                                   int64_t k, float* y_f32, uint16_t* y_bf16, void* stream) {
  const char* name = "wq_gemm_smallM_int8";
  int rc = check_common(name, x, q, scale, true, n, k, y_f32, y_bf16, 16, m, -1, k, kI8mMaxBytes);
  if (rc) return rc;
  if ((reinterpret_cast<uintptr_t>(scale) & 1u) != 0) return fail(WQ_ERR_ALIGN, "%s: scale must be 2-byte aligned", name);
  if (n == 0) return WQ_OK;
  if ((rc = check_device())) return rc;
  hipStream_t s = (hipStream_t)stream;
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
  if (m == 1) return run_gemv<FmtInt8, 1>(a, s, name);
  if (use_valu(true, m, a.chunks)) return run_gemv_m<FmtInt8>(a, m, s, name);
  // (k == 0: no passes; every output is the empty sum, 0)
  if (use_claim_kernel_i8(n, k)) {
    switch (m) {
      case 2: return launch_i8m_claim<2>(a, s);
      case 3: return launch_i8m_claim<3>(a, s);
      case 4: return launch_i8m_claim<4>(a, s);
      case 5: return launch_i8m_claim<5>(a, s);
      case 6: return launch_i8m_claim<6>(a, s);
      case 7: return launch_i8m_claim<7>(a, s);
      default: return launch_i8m_claim<8>(a, s);
    }
  }
  switch (m) {
    case 2: return launch_i8m<2>(a, s);
    case 3: return launch_i8m<3>(a, s);
    case 4: return launch_i8m<4>(a, s);
    case 5: return launch_i8m<5>(a, s);
    case 6: return launch_i8m<6>(a, s);
    case 7: return launch_i8m<7>(a, s);
    default: return launch_i8m<8>(a, s);
  }
}
