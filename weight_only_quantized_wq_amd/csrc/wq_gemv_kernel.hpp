// Streaming matvec kernel template shared by every weight format.
//
// Work decomposition (one launch per weight matrix):
//   * a row of W is `chunks` 16-byte chunks; lane l of a wave owns chunks
//     (ks * CPL + j) * 64 + l, j < CPL, of every row it visits, so each
//     wave-wide load is 1 KiB of one row, contiguous;
//   * `split` waves (ks = 0 .. split-1) cover one row together when a row has
//     more chunks than one wave can hold activations for (split-K); their
//     partial sums meet in LDS in a fixed order;
//   * a workgroup holds `groups` such wave teams; each team takes U rows per
//     batch, and workgroups stride over batches;
//   * the activations of a lane's chunks are loaded once into registers and
//     reused for every row (they are the same for all rows of W);
//   * weights are read with buffer loads through per-row resources, so rows
//     past n and chunks past a row's end read as zero with no branches;
//   * with PF, the next batch's weights are requested before the current one
//     is reduced (two register buffers), and the first batch is requested
//     before the activations are staged, so HBM requests stay in flight
//     through the arithmetic;
//   * per row: fp32 accumulation per lane, a DPP wave reduction, the split-K
//     sum through LDS, then the epilogue (row scale for int8, fp32 and/or
//     bf16 stores).
// No atomics: every output is reduced in one fixed order, so results are
// bitwise reproducible.
#pragma once

#include <stdint.h>

#include "wq_formats.hpp"

namespace wq {

struct GemvArgs {
  const uint16_t* x;      // [m][k] bf16
  const uint8_t* w;       // n rows of row_bytes
  const uint16_t* scale;  // int8: [n] bf16 row scales
  const uint32_t* sz;     // int4: [n][chunks] (scale | zero << 16)
  float* y32;             // [m][n] or null
  uint16_t* y16;          // [m][n] or null
  int64_t n;
  int64_t k;
  int64_t row_bytes;
  int64_t batches;
  int64_t batch_begin;    // multi-matrix launches: first global batch of this matrix
  int32_t chunks;
  int32_t split;
  int32_t groups;
  int32_t cpl;            // multi-matrix launches: chunks per lane used (<= CPL)
  int32_t gshift;         // int4: log2(group / 32): chunk c's (scale, zero) word is sz[row][c >> gshift]
  int32_t rpp;            // one-token step: rows sharing a wave pass (short rows; 0 or 1 = one row per wave)
  int32_t wide;           // one-token step, rpp > 1: each lane takes up to U * CPL chunks of one row
                          // (instead of CPL chunks of each of U rows)
};

// int4 with one group per row (per-channel): a shift past any row's chunk
// count maps every chunk to the row's single (scale, zero) word.
constexpr int kPerRowShift = 30;

// (scale, zero) words of an int4 row: chunks / 2^gshift, rounded up (one
// word for a per-row group).
__host__ __device__ inline int64_t int4_row_words(int64_t chunks, int gshift) {
  return (chunks + ((int64_t)1 << gshift) - 1) >> gshift;
}

template <class F, int U, int CPL>
struct Batch {
  u32x4 w[U][CPL];
  uint32_t aux[U][CPL];
  uint32_t sb;   // formats with a row scale: raw bf16 bits of this lane's output row (finish_batch)
};

// Requests batch b's weights through per-row buffer resources: a row past
// n gets an empty resource and a chunk past the row lies past the resource's
// end, so both read as zero without a branch.  off[j] = 16 * chunk index.
// The row scale the epilogue of lane l needs (row r0 + l / M) is requested
// with the batch, from a clamped row, so nothing waits for it inside the
// epilogue's branch.
template <class F, int U, int CPL, int M = 1>
__device__ __forceinline__ void load_batch(const GemvArgs& a, int64_t b, int rg, const uint32_t (&off)[CPL],
                                           Batch<F, U, CPL>& bt, int cpl = CPL) {
  const int64_t r0 = b * ((int64_t)a.groups * U) + (int64_t)rg * U;
  if constexpr (F::kRowScale) {
    const int lane = lane_id();
    int64_t rs = r0 + (lane < U * M ? lane / M : 0);
    if (rs >= a.n) rs = a.n - 1;
    bt.sb = (uint32_t)*gmem(a.scale + rs);
  } else {
    bt.sb = 0u;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r = r0 + u;
    const bool row_ok = r < a.n;
    const int64_t rr = row_ok ? r : 0;
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(a.w + rr * a.row_bytes, row_ok ? (uint32_t)a.row_bytes : 0u);
#pragma unroll
    for (int j = 0; j < CPL; ++j) bt.w[u][j] = j < cpl ? buffer_load16_nt(rw, off[j]) : u32x4{0, 0, 0, 0};
    if constexpr (F::kGroupAux) {
      const int64_t words = int4_row_words(a.chunks, a.gshift);
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.sz + rr * words, row_ok ? (uint32_t)words * 4u : 0u);
#pragma unroll
      for (int j = 0; j < CPL; ++j) bt.aux[u][j] = j < cpl ? buffer_load4_nt(rs, ((off[j] >> 4) >> a.gshift) << 2) : 0u;
    } else {
#pragma unroll
      for (int j = 0; j < CPL; ++j) bt.aux[u][j] = 0u;
    }
  }
}

// Reduces batch b (already loaded) and writes its outputs.
template <class F, int M, int CPL, int U, int WAVES>
__device__ __forceinline__ void finish_batch(const GemvArgs& a, int64_t b, int lane, int wave, int ks, int rg,
                                             const Batch<F, U, CPL>& bt, const typename F::X (&xr)[M][CPL],
                                             const float (&bias)[M], const typename F::K& kc,
                                             float (&red)[2][WAVES][U * M], int& buf, int cpl = CPL,
                                             bool active = true) {
  const int S = a.split;
  if (!active) {            // a wave with no row group in this matrix: barrier only
    if (S > 1) {
      __syncthreads();
      buf ^= 1;
    }
    return;
  }
  const int64_t r0 = b * ((int64_t)a.groups * U) + (int64_t)rg * U;
  float acc[U][M];
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int m = 0; m < M; ++m) acc[u][m] = bias[m];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      if (j >= cpl) break;
      typename F::D d;
      F::decode(bt.w[u][j], d, kc);
#pragma unroll
      for (int m = 0; m < M; ++m) acc[u][m] = F::dot(d, bt.aux[u][j], xr[m][j], acc[u][m]);
    }
  }

  float tot[U * M];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int m = 0; m < M; ++m) tot[u * M + m] = wave_sum(acc[u][m]);

  if (S > 1) {
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < U * M; ++i) red[buf][wave][i] = tot[i];
    }
    __syncthreads();
    if (ks == 0) {
#pragma unroll
      for (int i = 0; i < U * M; ++i) {
        float v = red[buf][rg * S][i];
        for (int s = 1; s < S; ++s) v += red[buf][rg * S + s][i];
        tot[i] = v;
      }
    }
    buf ^= 1;
  }

  if (ks == 0 && lane < U * M) {
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < U * M; ++i)
      if (lane == i) v = tot[i];
    const int u = lane / M;
    const int m = lane - u * M;
    const int64_t r = r0 + u;
    if (r < a.n) {
      if constexpr (F::kRowScale) v *= __uint_as_float(bt.sb << 16);
      if (a.y32) *gmem(a.y32 + (m * a.n + r)) = v;
      if (a.y16) *gmem(a.y16 + (m * a.n + r)) = f32_to_bf16(v);
    }
  }
}

template <class F, int M, int CPL, int U, int WAVES, bool PF>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(GemvArgs a) {
  const int lane = lane_id();
  const int wave = wave_id();
  const int ks = wave % a.split;
  const int rg = wave / a.split;

  int cidx[CPL];
  uint32_t off[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    cidx[j] = (ks * CPL + j) * kWave + lane;
    off[j] = (uint32_t)cidx[j] * 16u;
  }

  int64_t b = blockIdx.x;
  const int64_t step = gridDim.x;
  Batch<F, U, CPL> A;
  load_batch<F, U, CPL, M>(a, b, rg, off, A);

  typename F::X xr[M][CPL];
  float bias[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    bias[m] = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      xr[m][j] = F::load_x(a.x + m * a.k, cidx[j], cidx[j] < a.chunks);
      bias[m] += F::lane_bias(xr[m][j]);
    }
  }
  const typename F::K kc = F::consts();

  __shared__ float red[2][WAVES][U * M];
  int buf = 0;

  if constexpr (PF) {
    Batch<F, U, CPL> B;
    while (b < a.batches) {
      load_batch<F, U, CPL, M>(a, b + step, rg, off, B);
      finish_batch<F, M, CPL, U, WAVES>(a, b, lane, wave, ks, rg, A, xr, bias, kc, red, buf);
      b += step;
      if (b >= a.batches) break;
      load_batch<F, U, CPL, M>(a, b + step, rg, off, A);
      finish_batch<F, M, CPL, U, WAVES>(a, b, lane, wave, ks, rg, B, xr, bias, kc, red, buf);
      b += step;
    }
  } else {
    while (b < a.batches) {
      finish_batch<F, M, CPL, U, WAVES>(a, b, lane, wave, ks, rg, A, xr, bias, kc, red, buf);
      b += step;
      if (b < a.batches) load_batch<F, U, CPL, M>(a, b, rg, off, A);
    }
  }
}

}  // namespace wq
