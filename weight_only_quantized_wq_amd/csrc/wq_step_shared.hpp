// Decode-step kernel with the activations shared in LDS (one workgroup per CU).
//
// A batch-1 decode step streams every linear layer once.  This persistent
// kernel covers a whole step in one launch:
//   * each workgroup owns a contiguous range of the step's row batches, of
//     equal cost on the first launch and then proportional to its measured
//     speed (see StepBalance); one workgroup per CU, so waves of one CU never
//     compete across workgroups, whose issue priority follows dispatch order;
//   * per matrix segment of its range the workgroup stages that matrix's
//     activations ONCE into LDS in the format's pre-decoded form, so a single
//     wave can cover a row of any length -- no split-K, no cross-wave
//     reduction, no barrier inside a matrix; each wave claims its first
//     batches and requests their weights before the staging;
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

// LDS words for staged activations: 158 KiB of gfx950's 160 KiB per
// workgroup (one workgroup per CU), leaving room for the counter and the
// range.  With 17 words per 16 inputs (int8) a row of up to 36864 inputs
// stages whole.
constexpr int kSharedXWords = 40448;

// Chunks of one row the kernel can stage: the largest multiple of a pass
// (64 * CPL chunks) that fits the LDS budget.
template <class F, int CPL>
constexpr int shared_x_cmax() {
  return (kSharedXWords / F::kLdsWordsPerChunk) / (kWave * CPL) * (kWave * CPL);
}

// One batch-pass of weights in registers: U rows x CPL chunks (+ group words;
// packed short rows: + the row scale bits of the row the lane stores for u).
template <int U, int CPL>
struct PassBuf {
  u32x4 w[U][CPL];
  uint32_t aux[U][CPL];
  uint32_t sc[U];
};

// Claims the next batch index of the segment for the calling wave.
__device__ __forceinline__ int claim_batch(int* ctr, int lane) {
  int v = 0;
  if (lane == 0) v = atomicAdd(ctr, 1);
  return __builtin_amdgcn_readfirstlane(v);
}

// Loads one batch-pass; with !ok every load reads zeros (an empty resource)
// without touching memory.  The loads are issued either way, so the code
// after a conditional prefetch sees the same outstanding loads on every
// path and waits only for the pass it consumes.
template <class F, int U, int CPL>
__device__ __forceinline__ void load_pass(const GemvArgs& a, int64_t batch, int pass, int lane, PassBuf<U, CPL>& bt,
                                          bool ok = true) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r = batch * U + u;
    const bool row_ok = ok && r < a.n;
    const int64_t rr = row_ok ? r : 0;
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(a.w + rr * a.row_bytes, row_ok ? (uint32_t)a.row_bytes : 0u);
#pragma unroll
    for (int j = 0; j < CPL; ++j) bt.w[u][j] = buffer_load16_nt(rw, (uint32_t)(((pass * CPL + j) * kWave + lane) * 16));
    if constexpr (F::kGroupAux) {
      // chunk c's (scale, zero) word: c >> gshift of the row's words.  A
      // chunk past the row reads zero codes against zero activations, so it
      // adds nothing whichever word it reads (zero past the words, or a
      // per-row group's one word).
      const int64_t words = int4_row_words(a.chunks, a.gshift);
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.sz + rr * words, row_ok ? (uint32_t)words * 4u : 0u);
#pragma unroll
      for (int j = 0; j < CPL; ++j)
        bt.aux[u][j] = buffer_load4_nt(rs, (uint32_t)((((pass * CPL + j) * kWave + lane) >> a.gshift) * 4));
    } else {
#pragma unroll
      for (int j = 0; j < CPL; ++j) bt.aux[u][j] = 0u;
    }
  }
}

// Short rows (one pass of fewer than 64 * CPL / 2 chunks): R = a.rpp rows
// share a wave pass, L = 64 / R lanes each; lane (s, q) = (lane / L, lane % L)
// takes chunks q + j L of row (batch U + u) R + s.  One buffer resource spans
// the R rows (wave-uniform), and a chunk past its row reads an offset past
// the resource, so it neither reads the next row nor faults.
template <class F, int U, int CPL>
__device__ __forceinline__ void load_pass_packed(const GemvArgs& a, int64_t batch, int lane, PassBuf<U, CPL>& bt,
                                                 bool ok = true) {
  const int R = a.rpp, L = kWave / R;
  const int s = lane / L, q = lane - s * L;
  const uint32_t rb = (uint32_t)a.row_bytes;
  const int64_t words = int4_row_words(a.chunks, a.gshift);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r0 = (batch * U + u) * R;
    const int64_t left = a.n - r0;
    const uint32_t rows_ok = !ok || left <= 0 ? 0u : (left >= R ? (uint32_t)R : (uint32_t)left);
    const int64_t rr = rows_ok ? r0 : 0;
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(a.w + rr * a.row_bytes, rows_ok * rb);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = q + j * L;
      // wide passes (one row per lane): skip the slots past every lane's
      // chunks (wave-uniform); with U rows per lane every slot is in use
      if (U > 1 || j * L < a.chunks)
        bt.w[u][j] = buffer_load16_nt(rw, c < a.chunks ? (uint32_t)s * rb + (uint32_t)c * 16u : 0x80000000u);
    }
    if constexpr (F::kGroupAux) {
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.sz + rr * words, rows_ok * (uint32_t)words * 4u);
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = q + j * L;
        if (U > 1 || j * L < a.chunks)
          bt.aux[u][j] = buffer_load4_nt(
              rs, c < a.chunks ? ((uint32_t)s * (uint32_t)words + (uint32_t)(c >> a.gshift)) * 4u : 0x80000000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < CPL; ++j) bt.aux[u][j] = 0u;
    }
    if constexpr (F::kRowScale) {
      // requested with the pass, clamped to a valid row, so that nothing
      // waits for it before the next pass is requested
      int64_t r = r0 + s;
      if (r >= a.n) r = a.n - 1;
      bt.sc[u] = (uint32_t)*gmem(a.scale + r);
    }
  }
}

// Raw bf16 bits of the row scale of row batch * U + lane (formats with a
// row scale; clamped to a valid row, so the load needs no branch and nothing
// waits for it before the next pass is requested).
template <class F, int U>
__device__ __forceinline__ uint32_t row_scale_bits(const GemvArgs& a, int64_t batch, int lane) {
  if constexpr (F::kRowScale) {
    int64_t r = batch * U + (lane < U ? lane : 0);
    if (r >= a.n) r = a.n - 1;
    return (uint32_t)*gmem(a.scale + r);
  } else {
    return 0u;
  }
}

// Accumulates one batch-pass; after the row's last pass, reduces and stores
// (`sbits`: this lane's row_scale_bits of the batch).
template <class F, int U, int CPL, int CMAX>
__device__ __forceinline__ void finish_pass(const GemvArgs& a, int64_t batch, int pass, int passes, int lane,
                                            const PassBuf<U, CPL>& bt, const uint32_t* xs,
                                            const typename F::K& kc, float (&acc)[U], float bias, uint32_t sbits) {
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
      if constexpr (F::kRowScale) v *= __uint_as_float(sbits << 16);
      if (a.y32) *gmem(a.y32 + r) = v;
      if (a.y16) *gmem(a.y16 + r) = f32_to_bf16(v);
    }
  }
}

// Sum over the L lanes of a group (L a power of two, at most 32), the same
// tree in every group.
__device__ __forceinline__ float group_sum(float v, int L) {
  for (int o = L >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Accumulates a packed pass (load_pass_packed) and stores its U * R rows:
// the L lanes of each row are summed and lane q = 0 stores the row.
template <class F, int U, int CPL, int CMAX>
__device__ __forceinline__ void finish_pass_packed(const GemvArgs& a, int64_t batch, int lane,
                                                   const PassBuf<U, CPL>& bt, const uint32_t* xs,
                                                   const typename F::K& kc, float (&acc)[U], float bias) {
  const int R = a.rpp, L = kWave / R;
  const int s = lane / L, q = lane - s * L;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    if (U == 1 && j * L >= a.chunks) break;   // as loaded (load_pass_packed)
    const typename F::X xv = F::lds_x(xs, CMAX, q + j * L);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      typename F::D d;
      F::decode(bt.w[u][j], d, kc);
      acc[u] = F::dot(d, bt.aux[u][j], xv, acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float v = group_sum(acc[u], L);
    acc[u] = bias;
    const int64_t r = (batch * U + u) * R + s;
    if (q == 0 && r < a.n) {
      if constexpr (F::kRowScale) v *= __uint_as_float(bt.sc[u] << 16);
      if (a.y32) *gmem(a.y32 + r) = v;
      if (a.y16) *gmem(a.y16 + r) = f32_to_bf16(v);
    }
  }
}

// The packed segment loop: one pass per batch, the next batch's loads
// requested before the current one is reduced (two alternating buffers, as
// in stream_segment).
template <class F, int U, int CPL, int CMAX, class Stage>
__device__ __forceinline__ void stream_segment_packed(const GemvArgs& a, int64_t lb, int64_t le, const uint32_t* xs,
                                                      int* ctr, int lane, Stage&& stage) {
  const typename F::K kc = F::consts();
  int64_t cur = lb + claim_batch(ctr, lane);
  if (cur >= le) {
    stage();
    return;
  }
  PassBuf<U, CPL> A, B;
  load_pass_packed<F, U, CPL>(a, cur, lane, A);
  stage();
  float bias = 0.0f;
  if constexpr (F::kLaneBias) {
    const int L = kWave / a.rpp, q = lane % L;
    for (int j = 0; j < CPL; ++j) bias += F::lds_bias(xs, CMAX, q + j * L);
  }
  float acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = bias;
  for (;;) {
    int64_t nx = lb + claim_batch(ctr, lane);
    bool more = nx < le;
    load_pass_packed<F, U, CPL>(a, nx, lane, B, more);
    finish_pass_packed<F, U, CPL, CMAX>(a, cur, lane, A, xs, kc, acc, bias);
    if (!more) {
      wait_vmem_all();   // no path reaches the loop head with the last request in flight
      break;
    }
    cur = nx;
    nx = lb + claim_batch(ctr, lane);
    more = nx < le;
    load_pass_packed<F, U, CPL>(a, nx, lane, A, more);
    finish_pass_packed<F, U, CPL, CMAX>(a, cur, lane, B, xs, kc, acc, bias);
    if (!more) {
      wait_vmem_all();
      break;
    }
    cur = nx;
  }
}

// The waves' share of one matrix segment: batches [lb, le) of matrix `a`,
// claimed one at a time from `ctr` (zeroed before the segment starts).  A
// wave claims its first batches and requests their weights first, then
// calls `stage`, which stages the segment's activations in LDS `xs` and
// waits for the whole workgroup: the weights do not depend on the
// activations, so their latency runs under the staging.  Every wave calls
// `stage` exactly once, with or without a batch.  PACK: short rows, a.rpp of
// them per wave pass (one pass per batch).
template <class F, int U, int CPL, int CMAX, bool PF, bool PACK, class Stage>
__device__ __forceinline__ void stream_segment(const GemvArgs& a, int64_t lb, int64_t le, const uint32_t* xs,
                                               int* ctr, int lane, Stage&& stage) {
  if constexpr (PACK) {
    stream_segment_packed<F, U, CPL, CMAX>(a, lb, le, xs, ctr, lane, stage);
    return;
  }
  const int passes = a.cpl;
  const typename F::K kc = F::consts();
  int64_t cur = lb + claim_batch(ctr, lane);
  if (cur >= le) {
    stage();
    return;
  }
  int64_t nxt = lb + claim_batch(ctr, lane);
  PassBuf<U, CPL> A;
  load_pass<F, U, CPL>(a, cur, 0, lane, A);
  stage();
  float bias = 0.0f;
  if constexpr (F::kLaneBias) {
    for (int c = lane; c < passes * CPL * kWave; c += kWave) bias += F::lds_bias(xs, CMAX, c);
  }
  int pass = 0;
  float acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = bias;
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
      uint32_t sb = row_scale_bits<F, U>(a, cur, lane);
      load_pass<F, U, CPL>(a, c2, p2, lane, B, more);
      if (more && p2 == 0) nxt = lb + claim_batch(ctr, lane);
      finish_pass<F, U, CPL, CMAX>(a, cur, pass, passes, lane, A, xs, kc, acc, bias, sb);
      if (!more) {
        wait_vmem_all();   // no path reaches the loop head with the last request in flight
        break;
      }
      cur = c2;
      pass = p2;

      c2 = cur;
      p2 = pass + 1;
      if (p2 == passes) {
        c2 = nxt;
        p2 = 0;
      }
      more = c2 < le;
      sb = row_scale_bits<F, U>(a, cur, lane);
      load_pass<F, U, CPL>(a, c2, p2, lane, A, more);
      if (more && p2 == 0) nxt = lb + claim_batch(ctr, lane);
      finish_pass<F, U, CPL, CMAX>(a, cur, pass, passes, lane, B, xs, kc, acc, bias, sb);
      if (!more) {
        wait_vmem_all();
        break;
      }
      cur = c2;
      pass = p2;
    }
  } else {
    for (;;) {
      finish_pass<F, U, CPL, CMAX>(a, cur, pass, passes, lane, A, xs, kc, acc, bias,
                                   row_scale_bits<F, U>(a, cur, lane));
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

// Load balance across workgroups (one-token and int8 2..8-row steps).  A
// workgroup's time per unit of cost depends on what its range holds (rows
// of different lengths stream at different rates per byte; every matrix
// boundary inside a range costs a staging and a drain) and on the CU it runs
// on, and for a given plan it repeats from launch to launch: the workgroup
// -> CU assignment is stable and the ranges move little.  So each workgroup
// reports the cost of its range and the time it took, and a launch cuts with
// per-workgroup shares derived from the reports of the launch before the
// previous one.  Launch n (parity p = n & 1) reads shares[p] and writes
// reports[p]; the first of its workgroups to finish turns reports[p ^ 1]
// (launch n - 1, complete) into relative speeds and writes shares[p ^ 1]
// for launch n + 1, while the others are still streaming, so none of this
// work lengthens the launch; the last to finish only advances the launch
// count.  Nothing a launch reads is written during it.  The speeds move all
// the way to the first measurement, half and a third of the way for the
// second and third, a quarter for every later one; clamped to [0.5, 2],
// mean 1.  Every workgroup reads the same table, so the ranges always
// partition the step; which workgroup computes a row never changes the
// row's result.
constexpr int kStepMaxGroups = 8192;
struct StepBalance {
  int32_t done;                        // workgroups finished in this launch
  int32_t epoch;                       // launches of the plan so far (advanced by each launch's last workgroup)
  int32_t pad[2];
  float w[kStepMaxGroups];             // relative speed of workgroup g (mean 1 over the launch's workgroups)
  float cost[2][kStepMaxGroups];       // by launch parity: cost of workgroup g's range (units of the cut)
  float time[2][kStepMaxGroups];       // by launch parity: its duration (wall-clock ticks)
  double cum[2][kStepMaxGroups + 1];   // by launch parity: share of the step before workgroup g
};
static_assert(sizeof(StepBalance) % 16 == 0, "the verify state follows at a 16-byte boundary");

struct StepCuts {
  const double* prefix;   // [count + 1] cost of the step before matrix i
  const double* bcost;    // [count] cost of one batch of matrix i
  StepBalance* bal;
  int64_t total;          // batches in the step
  int32_t count;          // matrices
};

// A workgroup's balance report: agent-scope atomic stores or adds, then the
// `done` count; a later launch (per-workgroup speeds) or this launch's last
// workgroup (the verify kernel's long-row sums) reads them back with
// agent-scope atomic loads.  The only order needed is "report performed
// before the count", which a wait for this wave's outstanding memory
// operations gives; an agent-scope fence would add an L2 write-back and
// invalidate per workgroup (several microseconds at the end of every
// launch).  A report that came late would only blur one launch's factors:
// the cuts are valid for any factors.
__device__ __forceinline__ void report_in_order() { wait_vmem_all(); }

// Sum over the workgroup of one value per thread (NT threads).
template <int NT>
__device__ __forceinline__ double block_sum(double v, double* lds) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  __syncthreads();
  if (lane_id() == 0) lds[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) t += lds[i];
  return t;
}

// Sum of the values of the threads before this one (NT threads), and of all.
template <int NT>
__device__ __forceinline__ double block_exclusive_scan(double v, double* lds, double& all) {
  const int lane = lane_id();
  double inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const double o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  __syncthreads();
  if (lane == kWave - 1) lds[threadIdx.x >> 6] = inc;
  __syncthreads();
  double before = 0.0;
  all = 0.0;
  const int wv = (int)(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) {
    if (i < wv) before += lds[i];
    all += lds[i];
  }
  return before + inc - v;
}

// The first workgroup of a launch to finish (all NT threads): new speed
// weights from the reports in buffer `q` (measurement number `m` of the
// plan) and the cumulative shares written to buffer `q`, which the launch
// after this one cuts with.  Thread i handles workgroups [i * per,
// (i + 1) * per).  `lds`: NT / 64 doubles of LDS the workgroup no longer
// needs.
template <int NT>
__device__ __forceinline__ void step_balance_update(StepBalance* b, int G, int q, int m, double* lds) {
  constexpr int P = kStepMaxGroups / NT;
  const int per = (G + NT - 1) / NT;
  const int j0 = (int)threadIdx.x * per;
  float r[P], wv[P];
  double rs = 0.0, rn = 0.0;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    r[i] = 0.0f;
    wv[i] = 1.0f;
    const int j = j0 + i;
    if (i < per && j < G) {
      const float c = __hip_atomic_load(&b->cost[q][j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float t = __hip_atomic_load(&b->time[q][j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      wv[i] = __hip_atomic_load(&b->w[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      r[i] = (c > 0.0f && t > 0.0f) ? c / t : 0.0f;
      if (r[i] > 0.0f) {
        rs += r[i];
        rn += 1.0;
      }
    }
  }
  rs = block_sum<NT>(rs, lds);
  rn = block_sum<NT>(rn, lds);
  const float mean = rn > 0.0 ? (float)(rs / rn) : 0.0f;
  const float gain = m < 3 ? 1.0f / (float)(m + 1) : 0.25f;
  double local = 0.0;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    float v = wv[i];
    if (mean > 0.0f && r[i] > 0.0f) v = (1.0f - gain) * v + gain * (r[i] / mean);
    wv[i] = fminf(fmaxf(v, 0.5f), 2.0f);
    if (i < per && j0 + i < G) local += wv[i];
  }
  double all;
  double run = block_exclusive_scan<NT>(local, lds, all);
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int j = j0 + i;
    if (i < per && j < G) {
      run += wv[i];
      __hip_atomic_store(&b->w[j], (float)(wv[i] * (double)G / all), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&b->cum[q][j + 1], j + 1 == G ? 1.0 : run / all, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// This launch's number (read once at the start by every workgroup; only the
// launch's last workgroup changes it, after every workgroup has finished).
__device__ __forceinline__ int step_epoch(const StepBalance* b) { return __builtin_amdgcn_readfirstlane(b->epoch); }

// End of a balanced launch (every thread of the workgroup; `epoch` as read
// at its start): the workgroup reports the cost of its range (units of the
// cut) and the time since `t_start`.  The first workgroup to finish computes
// the shares of the launch after the next from the previous launch's
// reports; the last runs `on_last` (thread 0) and advances the launch
// count.  `lds`: WAVES doubles of LDS the workgroup no longer needs.
template <int WAVES, class OnLast>
__device__ __forceinline__ void step_balance_report(StepBalance* b, int epoch, double cost, long long t_start,
                                                    double* lds, OnLast&& on_last) {
  __shared__ int role;   // bit 0: first to finish, bit 1: last
  const int G = (int)gridDim.x;
  const int p = epoch & 1;
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_store(&b->cost[p][blockIdx.x], (float)cost, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&b->time[p][blockIdx.x], (float)(wall_clock64() - t_start), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    report_in_order();
    const int r = atomicAdd(&b->done, 1);
    role = (r == 0 ? 1 : 0) | (r == G - 1 ? 2 : 0);
    if (r == G - 1) {
      // every workgroup has reported (and read this launch's epoch)
      on_last();
      atomicExch(&b->done, 0);
      if (epoch < (1 << 30)) atomicExch(&b->epoch, epoch + 1);
    }
  }
  __syncthreads();
  if ((role & 1) && epoch >= 1) step_balance_update<WAVES * kWave>(b, G, p ^ 1, epoch - 1, lds);
}
template <int WAVES>
__device__ __forceinline__ void step_balance_report(StepBalance* b, int epoch, double cost, long long t_start,
                                                    double* lds) {
  step_balance_report<WAVES>(b, epoch, cost, t_start, lds, [] {});
}

// Workgroup g's share [c0, c1) of a launch of cost `total` (launch `epoch`).
__device__ __forceinline__ void step_share(const StepBalance* b, int epoch, double total, double& c0, double& c1) {
  const double* cum = b->cum[epoch & 1];
  c0 = total * cum[blockIdx.x];
  c1 = (int)blockIdx.x + 1 == (int)gridDim.x ? total : total * cum[blockIdx.x + 1];
}

// The persistent step's frame.  Each workgroup cuts its own contiguous range
// of the step's batches from the cost prefix and its share of the step
// (StepBalance), hands each matrix's part of it, batches [lb, le) of `a`, to
// `segment(a, lb, le)` (called by every thread of the workgroup), and then
// reports the cost it streamed and the time it took.
template <int WAVES, class Segment>
__device__ __forceinline__ void step_frame(const GemvArgs* __restrict__ mats, const StepCuts& cuts,
                                           Segment&& segment) {
  __shared__ int64_t range[2];
  __shared__ int first_mat;
  __shared__ double bal_lds[WAVES];
  const long long t_start = wall_clock64();
  const int epoch = step_epoch(cuts.bal);
  double c0, c1;
  step_share(cuts.bal, epoch, cuts.prefix[cuts.count], c0, c1);
  // the batch at cost c: first batch of matrix i (prefix[i] <= c < prefix[i + 1])
  // whose start is at or past c; every matrix is checked by one thread
  if (threadIdx.x == 0) {
    range[0] = cuts.total;
    range[1] = cuts.total;
    first_mat = cuts.count - 1;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < cuts.count; i += WAVES * kWave) {
    const double p0 = cuts.prefix[i], p1 = cuts.prefix[i + 1];
    const GemvArgs& m = mats[i];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const double c = e == 0 ? c0 : c1;
      if (p0 <= c && c < p1) {
        int64_t local = (int64_t)((c - p0) / cuts.bcost[i] + 0.999999);
        if (local > m.batches) local = m.batches;
        range[e] = m.batch_begin + local;
        if (e == 0) first_mat = i;
      }
    }
  }
  __syncthreads();
  int64_t gb = uniform_i64(range[0]);
  const int64_t gend = uniform_i64(range[1]);
  int mi = __builtin_amdgcn_readfirstlane(first_mat);
  while (gb < gend) {
    GemvArgs a = mats[mi];
    if (gb >= a.batch_begin + a.batches) {   // the range starts at the next matrix
      ++mi;
      continue;
    }
    const int64_t mend = a.batch_begin + a.batches;
    const int64_t lb = gb - a.batch_begin;
    const int64_t le = (gend < mend ? gend : mend) - a.batch_begin;
    segment(a, lb, le);
    gb = a.batch_begin + le;
    ++mi;
  }
  step_balance_report<WAVES>(cuts.bal, epoch, c1 - c0, t_start, bal_lds);
}

// mats: per-matrix descriptors (batch = U rows; `cpl` holds the number of
// passes per row).  Each segment's activations are staged in LDS, then the
// waves claim its batches one at a time.
template <class F, int U, int CPL, int WAVES, bool PF>
__global__ __launch_bounds__(WAVES * 64) void gemv_step_shared_kernel(const GemvArgs* __restrict__ mats,
                                                                      StepCuts cuts) {
  constexpr int CMAX = shared_x_cmax<F, CPL>();
  __shared__ __attribute__((aligned(16))) uint32_t xs[kSharedXWords];
  // batch counters of alternate segments: a segment's claims start before
  // its staging barrier, so its counter is cleared one segment ahead
  __shared__ int ctr[2];
  const int lane = lane_id();
  if (threadIdx.x < 2) ctr[threadIdx.x] = 0;
  int par = 0;
  step_frame<WAVES>(mats, cuts, [&](const GemvArgs& a, int64_t lb, int64_t le) {
    __syncthreads();   // every wave is done with the previous segment's LDS and counter
    if (threadIdx.x == 0) ctr[par ^ 1] = 0;
    auto stage = [&]() {
      const int cpad = a.cpl * CPL * kWave;
      for (int c = threadIdx.x; c < cpad; c += WAVES * kWave) F::stage(a.x, a.chunks, c, xs, CMAX);
      __syncthreads();
    };
    // wide passes for the formats whose activations are pre-decoded pairs
    // (int8's fp32 activations for four chunk slots of one row would not fit
    // the 16-wave register budget)
    if constexpr (!F::kRowScale) {
      if (a.rpp > 1 && a.wide) {
        stream_segment_packed<F, 1, U * CPL, CMAX>(a, lb, le, xs, &ctr[par], lane, stage);
        par ^= 1;
        return;
      }
    }
    if (a.rpp > 1)
      stream_segment<F, U, CPL, CMAX, PF, true>(a, lb, le, xs, &ctr[par], lane, stage);
    else
      stream_segment<F, U, CPL, CMAX, PF, false>(a, lb, le, xs, &ctr[par], lane, stage);
    par ^= 1;
  });
}

}  // namespace wq
