// Decode-step kernel with the activations shared in LDS (one workgroup per CU).
//
// A batch-1 decode step streams every linear layer once.  This persistent
// kernel covers a whole step in one launch:
//   * each workgroup owns a contiguous range of the step's row batches, cut
//     on the host so that every workgroup streams the same number of weight
//     bytes (one workgroup per CU: waves of one CU never compete across
//     workgroups, whose issue priority follows dispatch order);
//   * per matrix segment of its range the workgroup stages that matrix's
//     activations ONCE into LDS in the format's pre-decoded form, so a single
//     wave can cover a row of any length -- no split-K, no cross-wave
//     reduction, no barrier inside a matrix;
//   * the waves claim batches of U rows from an LDS counter, so a wave that
//     gets less issue time simply takes fewer batches;
//   * a row batch is streamed in passes of CPL 16-byte chunks per lane (64 *
//     CPL chunks per wave-wide pass, lane l taking chunks (p * CPL + j) * 64 +
//     l): with PF the next pass (of this batch or the next claimed one) is
//     requested before the current one is reduced, so HBM requests stay in
//     flight through the arithmetic;
//   * weights are read with nontemporal buffer loads through per-row
//     resources (rows past n and chunks past a row read as zero); LDS
//     activations past the row are staged as zeros;
//   * per row: fp32 accumulation per lane across passes, one DPP wave sum,
//     then the epilogue (fp32 and/or bf16 stores).
// The order of additions of a row depends only on its length, so outputs are
// bitwise reproducible whatever wave takes the row.
#pragma once

#include <stdint.h>

#include "wq_gemv_kernel.hpp"

namespace wq {

// LDS words for staged activations (64 KiB minus room for the counter).
constexpr int kSharedXWords = 16320;

// Chunks of one row the kernel can stage: the largest multiple of a pass
// (64 * CPL chunks) that fits the LDS budget.
template <class F, int CPL>
constexpr int shared_x_cmax() {
  return (kSharedXWords / F::kLdsWordsPerChunk) / (kWave * CPL) * (kWave * CPL);
}

// One batch-pass of weights in registers: U rows x CPL chunks (+ group words).
template <int U, int CPL>
struct PassBuf {
  u32x4 w[U][CPL];
  uint32_t aux[U][CPL];
};

// Claims the next batch index of the segment for the calling wave.
__device__ __forceinline__ int claim_batch(int* ctr, int lane) {
  int v = 0;
  if (lane == 0) v = atomicAdd(ctr, 1);
  return __builtin_amdgcn_readfirstlane(v);
}

template <class F, int U, int CPL>
__device__ __forceinline__ void load_pass(const GemvArgs& a, int64_t batch, int pass, int lane, PassBuf<U, CPL>& bt) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r = batch * U + u;
    const bool row_ok = r < a.n;
    const int64_t rr = row_ok ? r : 0;
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(a.w + rr * a.row_bytes, row_ok ? (uint32_t)a.row_bytes : 0u);
#pragma unroll
    for (int j = 0; j < CPL; ++j) bt.w[u][j] = buffer_load16_nt(rw, (uint32_t)(((pass * CPL + j) * kWave + lane) * 16));
    if constexpr (F::kGroupAux) {
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.sz + rr * a.chunks, row_ok ? (uint32_t)a.chunks * 4u : 0u);
#pragma unroll
      for (int j = 0; j < CPL; ++j) bt.aux[u][j] = buffer_load4_nt(rs, (uint32_t)(((pass * CPL + j) * kWave + lane) * 4));
    } else {
#pragma unroll
      for (int j = 0; j < CPL; ++j) bt.aux[u][j] = 0u;
    }
  }
}

// Accumulates one batch-pass; after the row's last pass, reduces and stores.
template <class F, int U, int CPL, int CMAX>
__device__ __forceinline__ void finish_pass(const GemvArgs& a, int64_t batch, int pass, int passes, int lane,
                                            const PassBuf<U, CPL>& bt, const uint32_t* xs,
                                            const typename F::K& kc, float (&acc)[U], float bias) {
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const typename F::X xv = F::lds_x(xs, CMAX, (pass * CPL + j) * kWave + lane);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      typename F::D d;
      F::decode(bt.w[u][j], d, kc);
      acc[u] = F::dot(d, bt.aux[u][j], xv, acc[u]);
    }
  }
  if (pass + 1 < passes) return;
  float tot[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    tot[u] = wave_sum(acc[u]);
    acc[u] = bias;
  }
  if (lane < U) {
    float v = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (lane == u) v = tot[u];
    const int64_t r = batch * U + lane;
    if (r < a.n) {
      if constexpr (F::kRowScale) v *= __uint_as_float((uint32_t)a.scale[r] << 16);
      if (a.y32) a.y32[r] = v;
      if (a.y16) a.y16[r] = f32_to_bf16(v);
    }
  }
}

// The waves' share of one matrix segment: batches [lb, le) of matrix `a`,
// claimed one at a time from `ctr` (zeroed by the caller).
template <class F, int U, int CPL, int CMAX, bool PF>
__device__ __forceinline__ void stream_segment(const GemvArgs& a, int64_t lb, int64_t le, const uint32_t* xs,
                                               int* ctr, int lane) {
  const int passes = a.cpl;
  const typename F::K kc = F::consts();
  float bias = 0.0f;
  if constexpr (F::kLaneBias) {
    for (int c = lane; c < passes * CPL * kWave; c += kWave) bias += F::lds_bias(xs, CMAX, c);
  }
  int64_t cur = lb + claim_batch(ctr, lane);
  if (cur >= le) return;
  int64_t nxt = lb + claim_batch(ctr, lane);
  int pass = 0;
  float acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = bias;
  PassBuf<U, CPL> A;
  load_pass<F, U, CPL>(a, cur, 0, lane, A);
  if constexpr (PF) {
    PassBuf<U, CPL> B;
    for (;;) {
      // the item after `cur/pass`: the next pass of this batch, or the
      // first pass of the batch claimed last
      int64_t c2 = cur;
      int p2 = pass + 1;
      if (p2 == passes) {
        c2 = nxt;
        p2 = 0;
      }
      bool more = c2 < le;
      if (more) load_pass<F, U, CPL>(a, c2, p2, lane, B);
      if (more && p2 == 0) nxt = lb + claim_batch(ctr, lane);
      finish_pass<F, U, CPL, CMAX>(a, cur, pass, passes, lane, A, xs, kc, acc, bias);
      if (!more) break;
      cur = c2;
      pass = p2;

      c2 = cur;
      p2 = pass + 1;
      if (p2 == passes) {
        c2 = nxt;
        p2 = 0;
      }
      more = c2 < le;
      if (more) load_pass<F, U, CPL>(a, c2, p2, lane, A);
      if (more && p2 == 0) nxt = lb + claim_batch(ctr, lane);
      finish_pass<F, U, CPL, CMAX>(a, cur, pass, passes, lane, B, xs, kc, acc, bias);
      if (!more) break;
      cur = c2;
      pass = p2;
    }
  } else {
    for (;;) {
      finish_pass<F, U, CPL, CMAX>(a, cur, pass, passes, lane, A, xs, kc, acc, bias);
      if (++pass == passes) {
        pass = 0;
        cur = nxt;
        if (cur >= le) break;
        nxt = lb + claim_batch(ctr, lane);
      }
      load_pass<F, U, CPL>(a, cur, pass, lane, A);
    }
  }
}

// mats: per-matrix descriptors (batch = U rows; `cpl` holds the number of
// passes per row); wg_begin[g] .. wg_begin[g + 1]: workgroup g's global
// batches, starting in matrix wg_mat[g].
template <class F, int U, int CPL, int WAVES, bool PF>
__global__ __launch_bounds__(WAVES * 64) void gemv_step_shared_kernel(const GemvArgs* __restrict__ mats,
                                                                      const int64_t* __restrict__ wg_begin,
                                                                      const int32_t* __restrict__ wg_mat) {
  constexpr int CMAX = shared_x_cmax<F, CPL>();
  __shared__ __attribute__((aligned(16))) uint32_t xs[kSharedXWords];
  __shared__ int ctr;
  const int lane = lane_id();
  int64_t gb = wg_begin[blockIdx.x];
  const int64_t gend = wg_begin[blockIdx.x + 1];
  int mi = wg_mat[blockIdx.x];
  while (gb < gend) {
    const GemvArgs a = mats[mi];
    const int64_t mend = a.batch_begin + a.batches;
    const int64_t lb = gb - a.batch_begin;
    const int64_t le = (gend < mend ? gend : mend) - a.batch_begin;
    const int cpad = a.cpl * CPL * kWave;
    __syncthreads();   // every wave is done with the previous segment's LDS
    for (int c = threadIdx.x; c < cpad; c += WAVES * kWave) F::stage(a.x, a.chunks, c, xs, CMAX);
    if (threadIdx.x == 0) ctr = 0;
    __syncthreads();
    stream_segment<F, U, CPL, CMAX, PF>(a, lb, le, xs, &ctr, lane);
    gb = a.batch_begin + le;
    ++mi;
  }
}

}  // namespace wq
