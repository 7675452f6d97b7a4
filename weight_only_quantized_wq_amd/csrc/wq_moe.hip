// Top-2 MoE decode step for one token with int8 per-row experts (Mixtral
// 8x7B shape), as two streaming launches on the caller's stream:
//
//   1. moe_w13_kernel: every workgroup routes (softmax top-2 of the logits,
//      equal logits -> lower index; gates renormalised over the pair), then
//      streams rows j and j + f of W13 for each selected expert and writes
//      a[slot][j] = silu(h_j) * h_{j+f} (fp32) to the caller's workspace.
//   2. moe_w2_kernel: two wave teams per workgroup, one per selected expert,
//      stream row n of their expert's W2 against that expert's a; the
//      workgroup combines y[n] = g_a o_a[n] + g_b o_b[n].
//
// Only the selected experts' weights are read and no host synchronisation is
// needed: the routing decision is recomputed (identically) on the device by
// every workgroup from the 8 logits.
#include <stdint.h>

#include "wq_formats.hpp"
#include "wq_host.hpp"

namespace wq {

struct MoeArgs {
  const uint16_t* x;      // [dim] bf16
  const float* logits;    // [e]
  const int8_t* w13;      // [e][2f][dim]
  const uint16_t* s13;    // [e][2f]
  const int8_t* w2;       // [e][dim][f]
  const uint16_t* s2;     // [e][dim]
  float* work;            // [2][f]
  float* y32;             // [dim] or null
  uint16_t* y16;          // [dim] or null
  int32_t* sel;           // [2] or null
  float* gates;           // [2] or null
  int64_t dim;
  int64_t f;
  int64_t batches;
  int32_t e;
  int32_t chunks;         // 16-byte chunks per row of the launched matrix
  int32_t split;          // waves per row (split-K)
  int32_t groups;         // teams per workgroup
};

// Top-2 of the logits (equal values -> lower index) and the pair's
// renormalised softmax gates g_a = 1 / (1 + exp(l_b - l_a)), g_b = 1 - g_a.
__device__ __forceinline__ void route_top2(const float* logits, int e, int& a, int& b, float& ga, float& gb) {
  a = 0;
  for (int i = 1; i < e; ++i)
    if (logits[i] > logits[a]) a = i;
  b = (a == 0) ? 1 : 0;
  for (int i = 0; i < e; ++i)
    if (i != a && logits[i] > logits[b]) b = i;
  float t = expf(logits[b] - logits[a]);   // in (0, 1]
  ga = 1.0f / (1.0f + t);
  gb = t * ga;
}

// Stage 1: W13 of both selected experts, SwiGLU epilogue.  A team of
// `split` waves handles one (slot, j) unit per batch: rows j and j + f.
template <int CPL, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void moe_w13_kernel(MoeArgs a) {
  using F = FmtInt8;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int S = a.split;
  const int ks = wave % S;
  const int rg = wave / S;

  int ea, eb;
  float ga, gb;
  route_top2(a.logits, a.e, ea, eb, ga, gb);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (a.sel) {
      a.sel[0] = ea;
      a.sel[1] = eb;
    }
    if (a.gates) {
      a.gates[0] = ga;
      a.gates[1] = gb;
    }
  }

  int cidx[CPL];
  bool cok[CPL];
  F::X xr[CPL];
  float bias = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    cidx[j] = (ks * CPL + j) * kWave + lane;
    cok[j] = cidx[j] < a.chunks;
    xr[j] = F::load_x(a.x, cidx[j], cok[j]);
    bias += F::lane_bias(xr[j]);
  }

  __shared__ float red[2][WAVES][2];
  int buf = 0;
  const int64_t units = 2 * a.f;
  const int64_t rows13 = 2 * a.f;

  for (int64_t bt = blockIdx.x; bt < a.batches; bt += gridDim.x) {
    const int64_t unit = bt * a.groups + rg;
    const bool unit_ok = unit < units;
    const int slot = unit_ok ? (int)(unit / a.f) : 0;
    const int64_t jrow = unit_ok ? unit - (int64_t)slot * a.f : 0;
    const int ex = slot == 0 ? ea : eb;
    const int8_t* base = a.w13 + (int64_t)ex * rows13 * a.dim;

    u32x4 wv[2][CPL];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int8_t* row = base + (jrow + u * a.f) * a.dim;
#pragma unroll
      for (int j = 0; j < CPL; ++j)
        wv[u][j] = (unit_ok && cok[j]) ? load_stream16(row + (int64_t)cidx[j] * 16) : u32x4{0, 0, 0, 0};
    }
    float tot[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float acc = bias;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        F::D d;
        F::decode(wv[u][j], d, F::K{});
        acc = F::dot(d, 0u, xr[j], acc);
      }
      tot[u] = wave_sum(acc);
    }
    if (S > 1) {
      if (lane == 0) {
        red[buf][wave][0] = tot[0];
        red[buf][wave][1] = tot[1];
      }
      __syncthreads();
      if (ks == 0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float v = red[buf][rg * S][u];
          for (int s = 1; s < S; ++s) v += red[buf][rg * S + s][u];
          tot[u] = v;
        }
      }
      buf ^= 1;
    }
    if (ks == 0 && lane == 0 && unit_ok) {
      const uint16_t* sc = a.s13 + (int64_t)ex * rows13;
      float h1 = tot[0] * __uint_as_float((uint32_t)sc[jrow] << 16);
      float h3 = tot[1] * __uint_as_float((uint32_t)sc[jrow + a.f] << 16);
      float silu = h1 / (1.0f + expf(-h1));
      a.work[(int64_t)slot * a.f + jrow] = silu * h3;
    }
  }
}

// Stage 2: W2 of both selected experts.  Team 0 streams expert a, team 1
// expert b, each against its own fp32 activations; U rows per batch.
template <int CPL, int WAVES, int U>
__global__ __launch_bounds__(WAVES * 64) void moe_w2_kernel(MoeArgs a) {
  using F = FmtInt8;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int S = a.split;
  const int ks = wave % S;
  const int team = wave / S;   // 0 or 1

  int ea, eb;
  float ga, gb;
  route_top2(a.logits, a.e, ea, eb, ga, gb);
  const int ex = team == 0 ? ea : eb;
  const int8_t* base = a.w2 + (int64_t)ex * a.dim * a.f;
  const float* xin = a.work + (int64_t)team * a.f;

  int cidx[CPL];
  bool cok[CPL];
  F::X xr[CPL];
  float bias = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    cidx[j] = (ks * CPL + j) * kWave + lane;
    cok[j] = cidx[j] < a.chunks;
    xr[j] = F::load_x(xin, cidx[j], cok[j]);
    bias += F::lane_bias(xr[j]);
  }

  __shared__ float red[2][WAVES][U];
  int buf = 0;
  for (int64_t bt = blockIdx.x; bt < a.batches; bt += gridDim.x) {
    const int64_t r0 = bt * U;
    u32x4 wv[U][CPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r0 + u;
      const int8_t* row = base + r * a.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j)
        wv[u][j] = (r < a.dim && cok[j]) ? load_stream16(row + (int64_t)cidx[j] * 16) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc = bias;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        F::D d;
        F::decode(wv[u][j], d, F::K{});
        acc = F::dot(d, 0u, xr[j], acc);
      }
      float t = wave_sum(acc);
      if (lane == 0) red[buf][wave][u] = t;
    }
    __syncthreads();
    if (wave == 0 && lane < U) {
      const int64_t r = r0 + lane;
      if (r < a.dim) {
        float o[2];
#pragma unroll
        for (int tm = 0; tm < 2; ++tm) {
          float v = red[buf][tm * S][lane];
          for (int s = 1; s < S; ++s) v += red[buf][tm * S + s][lane];
          o[tm] = v;
        }
        float sa = __uint_as_float((uint32_t)a.s2[(int64_t)ea * a.dim + r] << 16);
        float sb = __uint_as_float((uint32_t)a.s2[(int64_t)eb * a.dim + r] << 16);
        float y = ga * (sa * o[0]) + gb * (sb * o[1]);
        if (a.y32) a.y32[r] = y;
        if (a.y16) a.y16[r] = f32_to_bf16(y);
      }
    }
    buf ^= 1;
  }
}

// ---------------------------------------------------------------------------
// Host side

template <class K>
static int launch_grid(K kern, const MoeArgs& a, int threads, hipStream_t stream, int& resident) {
  if (resident == 0) resident = resident_groups(reinterpret_cast<const void*>(kern), threads);
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
    static int res = 0;
    return launch_grid(moe_w13_kernel<4, 4>, a, a.split * a.groups * kWave, stream, res);
  }
  a.split = (int)s;
  a.groups = 8 / (int)s;
  a.batches = (2 * a.f + a.groups - 1) / a.groups;
  static int res = 0;
  return launch_grid(moe_w13_kernel<4, 8>, a, a.split * a.groups * kWave, stream, res);
}

// W2 plans: two teams of `split` waves; chunks per lane 7 (two waves per
// team cover 14336 inputs exactly) or 4.
static int launch_w2(MoeArgs a, hipStream_t stream) {
  constexpr int U = 2;
  a.batches = (a.dim + U - 1) / U;
  const int64_t c = a.chunks;
  const int64_t s7 = (c + 64 * 7 - 1) / (64 * 7);
  const int64_t s4 = (c + 64 * 4 - 1) / (64 * 4);
  const int64_t waste7 = s7 * 64 * 7 - c, waste4 = s4 * 64 * 4 - c;
  if (s7 <= 2 && waste7 <= waste4) {
    a.split = (int)(s7 < 1 ? 1 : s7);
    a.groups = 2;
    static int res = 0;
    return launch_grid(moe_w2_kernel<7, 4, U>, a, 2 * a.split * kWave, stream, res);
  }
  if (s4 <= 8) {
    a.split = (int)(s4 < 1 ? 1 : s4);
    a.groups = 2;
    static int res = 0;
    return launch_grid(moe_w2_kernel<4, 16, U>, a, 2 * a.split * kWave, stream, res);
  }
  return fail(WQ_ERR_SHAPE, "moe_top2_gemv: f = %lld too large", (long long)a.f);
}

}  // namespace wq

using namespace wq;

extern "C" int moe_top2_gemv(const uint16_t* x, const float* logits, int64_t e, const int8_t* w13,
                             const uint16_t* s13, const int8_t* w2, const uint16_t* s2, int64_t dim, int64_t f,
                             float* work, float* y_f32, uint16_t* y_bf16, int32_t* sel, float* gates,
                             void* stream) {
  const char* name = "moe_top2_gemv";
  if (!x || !logits || !w13 || !s13 || !w2 || !s2 || !work)
    return fail(WQ_ERR_NULL, "%s: x, logits, w13, s13, w2, s2 and work must be non-null", name);
  if (!y_f32 && !y_bf16) return fail(WQ_ERR_NULL, "%s: at least one of y_f32 / y_bf16 must be non-null", name);
  if (e != 8) return fail(WQ_ERR_SHAPE, "%s: e = %lld; only 8 experts (top-2) are supported", name, (long long)e);
  if (dim < 16 || f < 16 || dim % 16 || f % 16 || dim > 32768 || f > 32768)
    return fail(WQ_ERR_SHAPE, "%s: dim = %lld, f = %lld must be multiples of 16 in [16, 32768]", name,
                (long long)dim, (long long)f);
  if (!aligned16(x) || !aligned16(w13) || !aligned16(w2) || !aligned16(work))
    return fail(WQ_ERR_ALIGN, "%s: x, w13, w2 and work must be 16-byte aligned", name);
  int rc = check_device();
  if (rc) return rc;
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
  if ((rc = launch_w13(a, s))) return rc;
  a.chunks = (int32_t)(f / 16);
  return launch_w2(a, s);
}
