// Top-2 MoE decode kernels (int8 per-row experts): routing, the W13 pass
// with its SwiGLU epilogue and the W2 pass with the gated combine.  The entry
// point and launch planning are in wq_moe.hip.
#pragma once

#include <stdint.h>

#include "wq_formats.hpp"

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
__device__ __forceinline__ void route_top2(const float* logits_ptr, int e, int& a, int& b, float& ga, float& gb) {
  const __attribute__((address_space(1))) float* logits = gmem(logits_ptr);
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
// Weights stream through per-row buffer resources (a unit past the end gets
// an empty resource; chunks past the row read as zero); with PF the next
// batch's loads are in flight while the current one is reduced.
template <int CPL>
struct W13Batch {
  u32x4 w[2][CPL];
  uint32_t sc[2];   // raw bf16 scales of rows j and j + f (requested with the batch)
};

template <int CPL>
__device__ __forceinline__ void w13_load(const MoeArgs& a, int64_t bt, int rg, int ea, int eb,
                                         const uint32_t (&off)[CPL], W13Batch<CPL>& B) {
  const int64_t unit = bt * a.groups + rg;
  const bool ok = unit < 2 * a.f;
  const int slot = ok ? (int)(unit / a.f) : 0;
  const int64_t jrow = ok ? unit - (int64_t)slot * a.f : 0;
  const int ex = slot == 0 ? ea : eb;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t row = (int64_t)ex * 2 * a.f + jrow + u * a.f;
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(a.w13 + row * a.dim, ok ? (uint32_t)a.dim : 0u);
#pragma unroll
    for (int j = 0; j < CPL; ++j) B.w[u][j] = buffer_load16_nt(r, off[j]);
    // the epilogue's scales, loaded here (a valid row also past the end) so
    // that nothing waits for them inside the epilogue's branch
    B.sc[u] = (uint32_t)a.s13[row];
  }
}

template <int CPL, int WAVES>
__device__ __forceinline__ void w13_finish(const MoeArgs& a, int64_t bt, int lane, int wave, int ks, int rg, int ea,
                                           int eb, const W13Batch<CPL>& B, const FmtInt8::X (&xr)[CPL], float bias,
                                           float (&red)[2][WAVES][2], int& buf) {
  using F = FmtInt8;
  const int S = a.split;
  float tot[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    float acc = bias;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      F::D d;
      F::decode(B.w[u][j], d, F::K{});
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
  const int64_t unit = bt * a.groups + rg;
  if (ks == 0 && lane == 0 && unit < 2 * a.f) {
    const int slot = (int)(unit / a.f);
    const int64_t jrow = unit - (int64_t)slot * a.f;
    float h1 = tot[0] * __uint_as_float(B.sc[0] << 16);
    float h3 = tot[1] * __uint_as_float(B.sc[1] << 16);
    float silu = h1 / (1.0f + expf(-h1));
    a.work[(int64_t)slot * a.f + jrow] = silu * h3;
  }
}

template <int CPL, int WAVES, bool PF>
__global__ __launch_bounds__(WAVES * 64) void moe_w13_kernel(MoeArgs a) {
  using F = FmtInt8;
  const int lane = lane_id();
  const int wave = wave_id();
  const int S = a.split;
  const int ks = wave % S;
  const int rg = wave / S;

  int ea, eb;
  float ga, gb;
  route_top2(a.logits, a.e, ea, eb, ga, gb);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (a.sel) {
      *gmem(a.sel + 0) = ea;
      *gmem(a.sel + 1) = eb;
    }
    if (a.gates) {
      *gmem(a.gates + 0) = ga;
      *gmem(a.gates + 1) = gb;
    }
  }

  int cidx[CPL];
  uint32_t off[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    cidx[j] = (ks * CPL + j) * kWave + lane;
    off[j] = (uint32_t)cidx[j] * 16u;
  }
  int64_t bt = blockIdx.x;
  const int64_t step = gridDim.x;
  W13Batch<CPL> A;
  w13_load<CPL>(a, bt, rg, ea, eb, off, A);

  F::X xr[CPL];
  float bias = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    xr[j] = F::load_x(a.x, cidx[j], cidx[j] < a.chunks);
    bias += F::lane_bias(xr[j]);
  }

  __shared__ float red[2][WAVES][2];
  int buf = 0;
  if constexpr (PF) {
    W13Batch<CPL> B;
    while (bt < a.batches) {
      w13_load<CPL>(a, bt + step, rg, ea, eb, off, B);
      w13_finish<CPL, WAVES>(a, bt, lane, wave, ks, rg, ea, eb, A, xr, bias, red, buf);
      bt += step;
      if (bt >= a.batches) break;
      w13_load<CPL>(a, bt + step, rg, ea, eb, off, A);
      w13_finish<CPL, WAVES>(a, bt, lane, wave, ks, rg, ea, eb, B, xr, bias, red, buf);
      bt += step;
    }
  } else {
    while (bt < a.batches) {
      w13_finish<CPL, WAVES>(a, bt, lane, wave, ks, rg, ea, eb, A, xr, bias, red, buf);
      bt += step;
      if (bt < a.batches) w13_load<CPL>(a, bt, rg, ea, eb, off, A);
    }
  }
}

// Stage 2: W2 of both selected experts.  Team 0 streams expert a, team 1
// expert b, each against its own fp32 activations; U rows per batch; the
// workgroup combines y[n] = g_a s_a[n] o_a[n] + g_b s_b[n] o_b[n].
template <int CPL, int U>
struct W2Batch {
  u32x4 w[U][CPL];
  uint32_t sc[2];   // raw bf16 scales of this lane's output row in experts a and b
};

template <int CPL, int U>
__device__ __forceinline__ void w2_load(const MoeArgs& a, int64_t bt, const int8_t* base, int ea, int eb,
                                        const uint32_t (&off)[CPL], W2Batch<CPL, U>& B) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r = bt * U + u;
    const bool ok = r < a.dim;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base + (ok ? r : 0) * a.f, ok ? (uint32_t)a.f : 0u);
#pragma unroll
    for (int j = 0; j < CPL; ++j) B.w[u][j] = buffer_load16_nt(rs, off[j]);
  }
  // the epilogue's scales (lane l < U: row bt U + l; clamped to a valid row)
  const int lane = lane_id();
  int64_t r = bt * U + (lane < U ? lane : 0);
  if (r >= a.dim) r = a.dim - 1;
  B.sc[0] = (uint32_t)a.s2[(int64_t)ea * a.dim + r];
  B.sc[1] = (uint32_t)a.s2[(int64_t)eb * a.dim + r];
}

template <int CPL, int WAVES, int U>
__device__ __forceinline__ void w2_finish(const MoeArgs& a, int64_t bt, int lane, int wave, int ea, int eb, float ga,
                                          float gb, const W2Batch<CPL, U>& B, const FmtInt8::X (&xr)[CPL],
                                          float bias, float (&red)[2][WAVES][U], int& buf) {
  using F = FmtInt8;
  const int S = a.split;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float acc = bias;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      F::D d;
      F::decode(B.w[u][j], d, F::K{});
      acc = F::dot(d, 0u, xr[j], acc);
    }
    const float t = wave_sum(acc);
    if (lane == 0) red[buf][wave][u] = t;
  }
  __syncthreads();
  if (wave == 0 && lane < U) {
    const int64_t r = bt * U + lane;
    if (r < a.dim) {
      float o[2];
#pragma unroll
      for (int tm = 0; tm < 2; ++tm) {
        float v = red[buf][tm * S][lane];
        for (int s = 1; s < S; ++s) v += red[buf][tm * S + s][lane];
        o[tm] = v;
      }
      const float sa = __uint_as_float(B.sc[0] << 16);
      const float sb = __uint_as_float(B.sc[1] << 16);
      const float y = ga * (sa * o[0]) + gb * (sb * o[1]);
      if (a.y32) *gmem(a.y32 + r) = y;
      if (a.y16) *gmem(a.y16 + r) = f32_to_bf16(y);
    }
  }
  buf ^= 1;
}

template <int CPL, int WAVES, int U, bool PF>
__global__ __launch_bounds__(WAVES * 64) void moe_w2_kernel(MoeArgs a) {
  using F = FmtInt8;
  const int lane = lane_id();
  const int wave = wave_id();
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
  uint32_t off[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    cidx[j] = (ks * CPL + j) * kWave + lane;
    off[j] = (uint32_t)cidx[j] * 16u;
  }
  int64_t bt = blockIdx.x;
  const int64_t step = gridDim.x;
  W2Batch<CPL, U> A;
  w2_load<CPL, U>(a, bt, base, ea, eb, off, A);

  F::X xr[CPL];
  float bias = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    xr[j] = F::load_x(xin, cidx[j], cidx[j] < a.chunks);
    bias += F::lane_bias(xr[j]);
  }

  __shared__ float red[2][WAVES][U];
  int buf = 0;
  if constexpr (PF) {
    W2Batch<CPL, U> B;
    while (bt < a.batches) {
      w2_load<CPL, U>(a, bt + step, base, ea, eb, off, B);
      w2_finish<CPL, WAVES, U>(a, bt, lane, wave, ea, eb, ga, gb, A, xr, bias, red, buf);
      bt += step;
      if (bt >= a.batches) break;
      w2_load<CPL, U>(a, bt + step, base, ea, eb, off, A);
      w2_finish<CPL, WAVES, U>(a, bt, lane, wave, ea, eb, ga, gb, B, xr, bias, red, buf);
      bt += step;
    }
  } else {
    while (bt < a.batches) {
      w2_finish<CPL, WAVES, U>(a, bt, lane, wave, ea, eb, ga, gb, A, xr, bias, red, buf);
      bt += step;
      if (bt < a.batches) w2_load<CPL, U>(a, bt, base, ea, eb, off, A);
    }
  }
}

}  // namespace wq
