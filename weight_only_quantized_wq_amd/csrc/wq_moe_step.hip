// Top-2 MoE decode over many layers: host planning and the two persistent
// launches (kernels in wq_moe_step.hpp).
#include <stdint.h>
#include <string.h>

#include <vector>

#include "wq_host.hpp"
#include "wq_moe_step.hpp"

namespace wq {

// Batch shapes (output units per wave batch, chunks per lane per pass,
// waves, prefetch), chosen by timing on the Mixtral 8x7B shape.
constexpr int kW13U = 2, kW13Cpl = 2, kW13Waves = 16;
constexpr bool kW13Pf = true;
constexpr int kW2U = 2, kW2Cpl = 2, kW2Waves = 16;
constexpr bool kW2Pf = true;

static const void* w13_kernel() {
  return reinterpret_cast<const void*>(moe_w13_step_kernel<kW13U, kW13Cpl, kW13Waves, kW13Pf>);
}
static const void* w2_kernel() {
  return reinterpret_cast<const void*>(moe_w2_step_kernel<kW2U, kW2Cpl, kW2Waves, kW2Pf>);
}

// Workspace: the layer descriptors, then the balance state of the W13
// launch and that of the W2 launch.
static int64_t desc_bytes(int32_t count) { return ((int64_t)count * (int64_t)sizeof(MoeLayerDesc) + 15) / 16 * 16; }

static int64_t grid_for(int resident, int64_t batches) {
  int64_t g = resident < 1 ? 1 : resident;
  if (g > batches) g = batches;
  return g < 1 ? 1 : g;
}

}  // namespace wq

using namespace wq;

extern "C" int64_t wq_moe_step_workspace_bytes(int32_t count) {
  if (count < 0) return 0;
  return desc_bytes(count) + 2 * (int64_t)sizeof(StepBalance);
}

extern "C" int wq_moe_step_prepare(int64_t e, int64_t dim, int64_t f, const wq_moe_layer* layers, int32_t count,
                                   void* workspace, int64_t workspace_bytes, wq_moe_plan* plan) {
  const char* name = "wq_moe_step_prepare";
  if (!layers || !workspace || !plan) return fail(WQ_ERR_NULL, "%s: layers, workspace and plan must be non-null", name);
  if (count < 1) return fail(WQ_ERR_SHAPE, "%s: count = %d must be >= 1", name, count);
  for (int32_t i = 0; i < count; ++i) {
    const wq_moe_layer& L = layers[i];
    if (!L.x || !L.logits || !L.w13 || !L.s13 || !L.w2 || !L.s2 || !L.work)
      return fail(WQ_ERR_NULL, "%s: layer %d: x, logits, w13, s13, w2, s2 and work must be non-null", name, i);
    if (!L.y_f32 && !L.y_bf16)
      return fail(WQ_ERR_NULL, "%s: layer %d: at least one of y_f32 / y_bf16 must be non-null", name, i);
  }
  if (e != 8) return fail(WQ_ERR_SHAPE, "%s: e = %lld; only 8 experts (top-2) are supported", name, (long long)e);
  constexpr int kMaxDim = moe_cmax<kW13Cpl, kMoeW13Words>() * 16;
  constexpr int kMaxF = moe_cmax<kW2Cpl, kMoeW2Words / 2>() * 16;
  if (dim < 16 || f < 16 || dim % 16 || f % 16 || dim > kMaxDim || f > kMaxF)
    return fail(WQ_ERR_SHAPE, "%s: dim = %lld, f = %lld must be multiples of 16 in [16, %d] and [16, %d]", name,
                (long long)dim, (long long)f, kMaxDim, kMaxF);
  for (int32_t i = 0; i < count; ++i) {
    const wq_moe_layer& L = layers[i];
    if (!aligned16(L.x) || !aligned16(L.w13) || !aligned16(L.w2) || !aligned16(L.work))
      return fail(WQ_ERR_ALIGN, "%s: layer %d: x, w13, w2 and work must be 16-byte aligned", name, i);
  }
  const int64_t need = wq_moe_step_workspace_bytes(count);
  if (workspace_bytes < need)
    return fail(WQ_ERR_SHAPE, "%s: workspace of %lld bytes is smaller than the %lld needed", name,
                (long long)workspace_bytes, (long long)need);
  if (!aligned16(workspace)) return fail(WQ_ERR_ALIGN, "%s: workspace must be 16-byte aligned", name);
  int rc = check_device();
  if (rc) return rc;

  std::vector<MoeLayerDesc> desc((size_t)count);
  for (int32_t i = 0; i < count; ++i) {
    const wq_moe_layer& L = layers[i];
    MoeLayerDesc& D = desc[(size_t)i];
    D.x = reinterpret_cast<const uint16_t*>(L.x);
    D.logits = L.logits;
    D.w13 = L.w13;
    D.s13 = L.s13;
    D.w2 = L.w2;
    D.s2 = L.s2;
    D.work = L.work;
    D.y32 = L.y_f32;
    D.y16 = L.y_bf16;
    D.sel = L.sel;
    D.gates = L.gates;
  }
  const int64_t b13 = (int64_t)count * 2 * ((f + kW13U - 1) / kW13U);
  const int64_t b2 = (int64_t)count * ((dim + kW2U - 1) / kW2U);
  int64_t grids[2] = {grid_for(resident_groups(w13_kernel(), kW13Waves * kWave), b13),
                      grid_for(resident_groups(w2_kernel(), kW2Waves * kWave), b2)};
  // descriptors, then both launches' balance states at equal shares
  std::vector<char> host((size_t)need, 0);
  memcpy(host.data(), desc.data(), desc.size() * sizeof(MoeLayerDesc));
  for (int l = 0; l < 2; ++l) {
    if (grids[l] > kStepMaxGroups) grids[l] = kStepMaxGroups;
    StepBalance* bal = reinterpret_cast<StepBalance*>(host.data() + desc_bytes(count) + l * sizeof(StepBalance));
    for (int64_t g = 0; g < grids[l]; ++g) bal->w[g] = 1.0f;
    for (int p = 0; p < 2; ++p) {
      for (int64_t g = 0; g < grids[l]; ++g) bal->cum[p][g] = (double)g / (double)grids[l];
      bal->cum[p][grids[l]] = 1.0;
    }
  }
  hipError_t err = hipMemcpy(workspace, host.data(), host.size(), hipMemcpyHostToDevice);
  if (err != hipSuccess) {
    (void)hipGetLastError();
    return fail(WQ_ERR_LAUNCH, "%s: copying the plan to the workspace failed: %s", name, hipGetErrorString(err));
  }
  memset(plan, 0, sizeof(*plan));
  plan->dim = dim;
  plan->f = f;
  plan->e = (int32_t)e;
  plan->count = count;
  plan->grid13 = (int32_t)grids[0];
  plan->grid2 = (int32_t)grids[1];
  plan->workspace = workspace;
  return WQ_OK;
}

extern "C" int wq_moe_step_run(const wq_moe_plan* plan, void* stream) {
  const char* name = "wq_moe_step_run";
  if (!plan || !plan->workspace) return fail(WQ_ERR_NULL, "%s: plan and its workspace must be non-null", name);
  if (plan->count < 1 || plan->e != 8 || plan->grid13 < 1 || plan->grid2 < 1 || plan->dim < 16 || plan->f < 16)
    return fail(WQ_ERR_SHAPE, "%s: the plan was not produced by wq_moe_step_prepare", name);
  int rc = check_device();
  if (rc) return rc;
  if (plan->grid13 > kStepMaxGroups || plan->grid2 > kStepMaxGroups)
    return fail(WQ_ERR_SHAPE, "%s: the plan was not produced by wq_moe_step_prepare", name);
  MoeStepDims d{plan->dim, plan->f, plan->e, plan->count};
  char* ws = reinterpret_cast<char*>(const_cast<void*>(plan->workspace));
  const MoeLayerDesc* L = reinterpret_cast<const MoeLayerDesc*>(ws);
  StepBalance* bal13 = reinterpret_cast<StepBalance*>(ws + desc_bytes(plan->count));
  StepBalance* bal2 = bal13 + 1;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL((moe_w13_step_kernel<kW13U, kW13Cpl, kW13Waves, kW13Pf>), dim3((unsigned)plan->grid13),
                     dim3(kW13Waves * kWave), 0, s, L, d, bal13);
  rc = launch_status(name);
  if (rc) return rc;
  hipLaunchKernelGGL((moe_w2_step_kernel<kW2U, kW2Cpl, kW2Waves, kW2Pf>), dim3((unsigned)plan->grid2),
                     dim3(kW2Waves * kWave), 0, s, L, d, bal2);
  return launch_status(name);
}
