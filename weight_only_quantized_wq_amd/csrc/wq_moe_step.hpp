// Top-2 MoE decode step over many layers in two persistent launches (int8
// per-row experts): all layers' W13 passes, then all layers' W2 passes.
//
// Every layer has its own token (x), router logits, experts, workspace and
// output; the layers do not feed each other, so the W13 pass of every layer
// can run in one launch and the W2 pass of every layer in a second one (the
// W2 pass of a layer reads the SwiGLU activations its W13 pass wrote).
//
// Both launches follow the shared-activation scheme of the decode step:
//   * one workgroup per CU owns a contiguous range of the launch's batches
//     (layer after layer; all layers have the same shape, so every batch
//     costs the same), equal in size on a plan's first launches and then
//     proportional to the workgroup's measured speed (StepBalance, one state
//     per launch);
//   * per layer segment the workgroup routes (softmax top-2 of the logits,
//     equal logits -> lower index, gates renormalised over the pair; every
//     workgroup derives the same choice) and stages the layer's activations
//     once into LDS as fp32 (x for W13; both experts' SwiGLU outputs for W2);
//   * waves claim batches from an LDS counter and stream whole rows in passes
//     of CPL 16-byte chunks per lane, the next pass requested before the
//     current one is reduced;
//   * W13 batch: U units j of one selected expert, each the row pair (j, j + f)
//     -> a[j] = silu(s_j h_j) * (s_{j+f} h_{j+f}) into the layer's workspace;
//   * W2 batch: U output rows n, each row n of both selected experts ->
//     y[n] = g_a (s_a[n] o_a[n]) + g_b (s_b[n] o_b[n]).
// Only the selected experts' weights are read.  Each row is reduced in an
// order that depends only on its length, so outputs are bitwise
// reproducible whichever wave takes a row.
#pragma once

#include <stdint.h>

#include "wq_moe_kernel.hpp"
#include "wq_step_shared.hpp"

namespace wq {

// Per-layer descriptor (device copy written by wq_moe_step_prepare).
struct MoeLayerDesc {
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
};

struct MoeStepDims {
  int64_t dim;
  int64_t f;
  int32_t e;
  int32_t count;   // layers
};

// LDS words for staged activations: W13 stages one x, W2 two expert inputs.
constexpr int kMoeW13Words = 16320;
constexpr int kMoeW2Words = 38400;

template <int CPL, int WORDS>
constexpr int moe_cmax() {
  return (WORDS / FmtInt8::kLdsWordsPerChunk) / (kWave * CPL) * (kWave * CPL);
}

template <int NR, int CPL>
struct MoePass {
  u32x4 w[NR][CPL];
};

// Loads pass `pass` of NR rows; row i starts at base[i] and has `row_bytes`
// bytes when ok[i] (otherwise it reads as zero).
template <int NR, int CPL>
__device__ __forceinline__ void moe_load_pass(const int8_t* const (&base)[NR], const bool (&ok)[NR], uint32_t row_bytes,
                                              int pass, int lane, MoePass<NR, CPL>& p) {
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(ok[i] ? base[i] : base[0], ok[i] ? row_bytes : 0u);
#pragma unroll
    for (int j = 0; j < CPL; ++j) p.w[i][j] = buffer_load16_nt(r, (uint32_t)(((pass * CPL + j) * kWave + lane) * 16));
  }
}

// Accumulates pass `pass` of NR rows; rows [q NR / PLANES, (q + 1) NR /
// PLANES) read the activation plane xs + q * PLANE (one plane's values are
// held in registers at a time).
template <int NR, int CPL, int CMAX, int PLANES>
__device__ __forceinline__ void moe_acc_pass(const MoePass<NR, CPL>& p, const uint32_t* xs, int pass, int lane,
                                             float (&acc)[NR]) {
  using F = FmtInt8;
  constexpr int PLANE = CMAX * F::kLdsWordsPerChunk;
  constexpr int RP = NR / PLANES;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = (pass * CPL + j) * kWave + lane;
#pragma unroll
    for (int q = 0; q < PLANES; ++q) {
      const F::X xv = F::lds_x(xs + q * PLANE, CMAX, c);
#pragma unroll
      for (int i = q * RP; i < (q + 1) * RP; ++i) {
        F::D d;
        F::decode(p.w[i][j], d, F::K{});
        acc[i] = F::dot(d, 0u, xv, acc[i]);
      }
    }
  }
}

// The waves' share of one layer segment: batches [lo, hi) claimed one at a
// time from `ctr`, each streamed in `passes` passes of NR rows.  The next
// pass (of this batch or of the batch claimed last) is requested before the
// current one is reduced; the two pass buffers alternate, so no loaded value
// is copied (a copy would wait for the loads just issued), and the request is
// issued on every path (empty rows when there is none), so each pass waits
// only for its own loads.  rows(b, base, ok) gives batch b's row pointers,
// scales(b) loads the two bf16 row scales the epilogue of batch b reads, as
// raw bits, from clamped (always valid) addresses without a branch -- so
// nothing waits for them before the next pass is requested -- and
// finish(b, acc, sc) reduces and stores a finished batch.
template <int NR, int CPL, int CMAX, int PLANES, class Rows, class Scales, class Finish>
__device__ __forceinline__ void moe_stream(int64_t lo, int64_t hi, int passes, uint32_t row_bytes, int* ctr,
                                           int lane, const uint32_t* xs, float (&acc)[NR], Rows&& rows,
                                           Scales&& scales, Finish&& finish) {
  int64_t cur = lo + claim_batch(ctr, lane);
  if (cur >= hi) return;
  int64_t nxt = lo + claim_batch(ctr, lane);
  int pass = 0;
  bool more = true;
  const int8_t* base[NR];
  bool ok[NR];
  rows(cur, base, ok);
  MoePass<NR, CPL> A, B;
  moe_load_pass<NR, CPL>(base, ok, row_bytes, 0, lane, A);
  auto step = [&](const MoePass<NR, CPL>& p, MoePass<NR, CPL>& nx) {
    const int64_t c_batch = cur;
    const int c_pass = pass;
    int64_t c2 = cur;
    int p2 = pass + 1;
    if (p2 == passes) {
      c2 = nxt;
      p2 = 0;
    }
    more = c2 < hi;
    const bool last = c_pass + 1 == passes;
    const uint2 sc = scales(c_batch);   // every pass: a branch would make the loads wait at its end
    if (more && p2 == 0) rows(c2, base, ok);
    bool live[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) live[i] = more && ok[i];
    moe_load_pass<NR, CPL>(base, live, row_bytes, p2, lane, nx);
    if (more && p2 == 0) nxt = lo + claim_batch(ctr, lane);
    moe_acc_pass<NR, CPL, CMAX, PLANES>(p, xs, c_pass, lane, acc);
    if (last) finish(c_batch, acc, sc);
    cur = c2;
    pass = p2;
  };
  // the request left in flight is drained on the way out, so that no path
  // reaches the loop head with loads outstanding
  for (;;) {
    step(A, B);
    if (!more) {
      wait_vmem_all();
      break;
    }
    step(B, A);
    if (!more) {
      wait_vmem_all();
      break;
    }
  }
}

// Workgroup range [lo, hi) of a launch of `total` batches.
// This workgroup's batches [lo, hi) of `total` (launch `epoch`), from its
// share of the launch: neighbours round their common boundary the same way.
__device__ __forceinline__ void moe_range(const StepBalance* b, int epoch, int64_t total, int64_t& lo, int64_t& hi,
                                          double& cost) {
  double c0, c1;
  step_share(b, epoch, (double)total, c0, c1);
  lo = (int64_t)(c0 + 0.5);
  hi = (int)blockIdx.x + 1 == (int)gridDim.x ? total : (int64_t)(c1 + 0.5);
  if (lo > total) lo = total;
  if (hi > total) hi = total;
  if (hi < lo) hi = lo;
  cost = c1 - c0;
}

// ---------------------------------------------------------------------------
// Launch 1: W13 of every layer.

template <int U, int CPL, int WAVES, bool PF>
__global__ __launch_bounds__(WAVES * 64) void moe_w13_step_kernel(const MoeLayerDesc* __restrict__ layers,
                                                                   MoeStepDims d, StepBalance* bal) {
  constexpr int CMAX = moe_cmax<CPL, kMoeW13Words>();
  constexpr int NR = 2 * U;
  __shared__ __attribute__((aligned(16))) uint32_t xs[kMoeW13Words];
  __shared__ int ctr;
  __shared__ double bal_lds[WAVES];
  const long long t_start = wall_clock64();
  const int epoch = step_epoch(bal);
  const int lane = lane_id();
  const int chunks = (int)(d.dim / 16);
  const int passes = (chunks + CPL * kWave - 1) / (CPL * kWave);
  const int64_t half = (d.f + U - 1) / U;   // batches per selected expert
  const int64_t per_layer = 2 * half;
  int64_t gb, gend;
  double cost;
  moe_range(bal, epoch, per_layer * d.count, gb, gend, cost);
  while (gb < gend) {
    const int layer = (int)(gb / per_layer);
    const int64_t lo = gb - (int64_t)layer * per_layer;
    const int64_t hi = gend - (int64_t)layer * per_layer < per_layer ? gend - (int64_t)layer * per_layer : per_layer;
    const MoeLayerDesc L = layers[layer];
    int ea, eb;
    float ga, gbt;
    route_top2(L.logits, d.e, ea, eb, ga, gbt);
    __syncthreads();   // the previous segment's LDS reads are done
    for (int c = threadIdx.x; c < passes * CPL * kWave; c += WAVES * kWave) FmtInt8::stage(L.x, chunks, c, xs, CMAX);
    if (threadIdx.x == 0) {
      ctr = 0;
      if (lo == 0) {
        if (L.sel) {
          *gmem(L.sel + 0) = ea;
          *gmem(L.sel + 1) = eb;
        }
        if (L.gates) {
          *gmem(L.gates + 0) = ga;
          *gmem(L.gates + 1) = gbt;
        }
      }
    }
    __syncthreads();
    float bias = 0.0f;
    if constexpr (FmtInt8::kLaneBias)
      for (int c = lane; c < passes * CPL * kWave; c += kWave) bias += FmtInt8::lds_bias(xs, CMAX, c);

    // batch b: units j0 .. j0 + U - 1 of expert slot b / half
    auto rows = [&](int64_t b, const int8_t* (&base)[NR], bool (&ok)[NR]) {
      const int slot = b >= half ? 1 : 0;   // b < 2 half
      const int64_t j0 = (b - slot * half) * U;
      const int ex = slot == 0 ? ea : eb;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = j0 + u;
        ok[u] = ok[U + u] = j < d.f;
        const int64_t r1 = (int64_t)ex * 2 * d.f + (j < d.f ? j : 0);
        base[u] = L.w13 + r1 * d.dim;
        base[U + u] = L.w13 + (r1 + d.f) * d.dim;
      }
    };
    // this lane's (w1, w3) row scales of batch b (lanes < U)
    auto scales = [&](int64_t b) -> uint2 {
      const int slot = b >= half ? 1 : 0;   // b < 2 half
      int64_t j = (b - slot * half) * U + lane;
      if (j >= d.f) j = d.f - 1;
      const int ex = slot == 0 ? ea : eb;
      const __attribute__((address_space(1))) uint16_t* sc = gmem(L.s13 + (int64_t)ex * 2 * d.f);
      return uint2{(uint32_t)sc[j], (uint32_t)sc[j + d.f]};
    };
    auto finish = [&](int64_t b, float (&acc)[NR], uint2 sc) {
      float tot[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        tot[i] = wave_sum(acc[i]);
        acc[i] = bias;
      }
      const int slot = b >= half ? 1 : 0;   // b < 2 half
      const int64_t j0 = (b - slot * half) * U;
      if (lane < U && j0 + lane < d.f) {
        float h1 = 0.0f, h3 = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (lane == u) {
            h1 = tot[u];
            h3 = tot[U + u];
          }
        const int64_t j = j0 + lane;
        h1 *= __uint_as_float(sc.x << 16);
        h3 *= __uint_as_float(sc.y << 16);
        *gmem(L.work + ((int64_t)slot * d.f + j)) = h1 / (1.0f + expf(-h1)) * h3;
      }
    };

    float acc[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) acc[i] = bias;
    moe_stream<NR, CPL, CMAX, 1>(lo, hi, passes, (uint32_t)d.dim, &ctr, lane, xs, acc, rows, scales, finish);
    gb = (int64_t)layer * per_layer + hi;
  }
  step_balance_report<WAVES>(bal, epoch, cost, t_start, bal_lds);
}

// ---------------------------------------------------------------------------
// Launch 2: W2 of every layer with the gated combine.

template <int U, int CPL, int WAVES, bool PF>
__global__ __launch_bounds__(WAVES * 64) void moe_w2_step_kernel(const MoeLayerDesc* __restrict__ layers,
                                                                  MoeStepDims d, StepBalance* bal) {
  constexpr int CMAX = moe_cmax<CPL, kMoeW2Words / 2>();
  constexpr int PLANE = CMAX * FmtInt8::kLdsWordsPerChunk;
  constexpr int NR = 2 * U;
  __shared__ __attribute__((aligned(16))) uint32_t xs[kMoeW2Words];
  __shared__ int ctr;
  __shared__ double bal_lds[WAVES];
  const long long t_start = wall_clock64();
  const int epoch = step_epoch(bal);
  const int lane = lane_id();
  const int chunks = (int)(d.f / 16);
  const int passes = (chunks + CPL * kWave - 1) / (CPL * kWave);
  const int64_t per_layer = (d.dim + U - 1) / U;
  int64_t gb, gend;
  double cost;
  moe_range(bal, epoch, per_layer * d.count, gb, gend, cost);
  while (gb < gend) {
    const int layer = (int)(gb / per_layer);
    const int64_t lo = gb - (int64_t)layer * per_layer;
    const int64_t hi = gend - (int64_t)layer * per_layer < per_layer ? gend - (int64_t)layer * per_layer : per_layer;
    const MoeLayerDesc L = layers[layer];
    int ea, eb;
    float ga, gbt;
    route_top2(L.logits, d.e, ea, eb, ga, gbt);
    __syncthreads();
    for (int c = threadIdx.x; c < passes * CPL * kWave; c += WAVES * kWave) {
      FmtInt8::stage(L.work, chunks, c, xs, CMAX);
      FmtInt8::stage(L.work + d.f, chunks, c, xs + PLANE, CMAX);
    }
    if (threadIdx.x == 0) ctr = 0;
    __syncthreads();
    float bias[2] = {0.0f, 0.0f};
    if constexpr (FmtInt8::kLaneBias) {
      for (int c = lane; c < passes * CPL * kWave; c += kWave) {
        bias[0] += FmtInt8::lds_bias(xs, CMAX, c);
        bias[1] += FmtInt8::lds_bias(xs + PLANE, CMAX, c);
      }
    }

    // batch b: output rows n0 .. n0 + U - 1, row n of expert a (rows 0..U-1)
    // and of expert b (rows U..2U-1)
    auto rows = [&](int64_t b, const int8_t* (&base)[NR], bool (&ok)[NR]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t n = b * U + u;
        ok[u] = ok[U + u] = n < d.dim;
        const int64_t nn = n < d.dim ? n : 0;
        base[u] = L.w2 + ((int64_t)ea * d.dim + nn) * d.f;
        base[U + u] = L.w2 + ((int64_t)eb * d.dim + nn) * d.f;
      }
    };
    // this lane's row scales of batch b in experts a and b (lanes < U)
    auto scales = [&](int64_t b) -> uint2 {
      int64_t n = b * U + lane;
      if (n >= d.dim) n = d.dim - 1;
      return uint2{(uint32_t)*gmem(L.s2 + ((int64_t)ea * d.dim + n)), (uint32_t)*gmem(L.s2 + ((int64_t)eb * d.dim + n))};
    };
    auto finish = [&](int64_t b, float (&acc)[NR], uint2 sc) {
      float tot[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        tot[i] = wave_sum(acc[i]);
        acc[i] = bias[i < U ? 0 : 1];
      }
      const int64_t n = b * U + lane;
      if (lane < U && n < d.dim) {
        float oa = 0.0f, ob = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (lane == u) {
            oa = tot[u];
            ob = tot[U + u];
          }
        const float y = ga * (__uint_as_float(sc.x << 16) * oa) + gbt * (__uint_as_float(sc.y << 16) * ob);
        if (L.y32) *gmem(L.y32 + n) = y;
        if (L.y16) *gmem(L.y16 + n) = f32_to_bf16(y);
      }
    };

    float acc[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) acc[i] = bias[i < U ? 0 : 1];
    moe_stream<NR, CPL, CMAX, 2>(lo, hi, passes, (uint32_t)d.f, &ctr, lane, xs, acc, rows, scales, finish);
    gb = (int64_t)layer * per_layer + hi;
  }
  step_balance_report<WAVES>(bal, epoch, cost, t_start, bal_lds);
}

}  // namespace wq
