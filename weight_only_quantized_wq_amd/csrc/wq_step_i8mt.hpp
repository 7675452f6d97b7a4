// 2..8 token rows through int8 weights (one bf16 scale per output row) on
// the matrix cores, v_mfma_f32_16x16x32_bf16, for the decode step and for
// one matrix:
//   * A = 16 weight rows x 32 inputs: lane l holds row l % 16, inputs
//     8 (l / 16) .. + 7 of the MFMA's K slice.  Each code becomes an exact
//     bf16 (a signed 8-bit integer has at most 8 significant bits): a
//     sign-extending byte conversion to fp32, whose upper half is the bf16.
//   * B = the token rows' activations: column t is token t (zero for t >= M),
//     read straight from memory -- the same M x K values serve every tile of
//     the matrix, so they stay in L2.
//   * D[row][t] accumulates in fp32 over the whole row; y = scale * D.
// A wave streams a batch of U tiles (16 U rows) over K in passes of 128
// inputs (bytes) per row.  The A layout puts 16 rows in the lanes of one
// register, but a load instruction reaches full HBM rate only when it reads
// whole 128-byte lines: with 64 bytes of each of 16 rows per instruction a
// pure stream of this shape runs at ~70 % of peak, with 128 bytes of each of
// 8 rows at ~87 %.  So a tile-pass is loaded as two instructions of 8 rows x
// 128 bytes (lane l: row l / 8 (+ 8), bytes 16 (l % 8) .. + 15), stored into
// a per-wave LDS tile and read back in the A layout: MFMA m of the pass takes
// bytes 32 m + 8 s .. + 7 of its row in k-slot s.  The 16-byte slots of a
// row are XOR-swizzled (slot p of row r at p ^ (r / 2 % 8)): rows 2 i and
// 2 i + 1 fill the two halves of one 256-byte bank span, so the stores (two
// rows of 8 slots per 16 lanes) and the 8-byte reads (one slot of 16 rows)
// fall in distinct banks.  The MACs cost one MFMA per 512 weight bytes, the
// decode 1.5 VALU ops per byte.
#pragma once

#include <stdint.h>

#include "wq_claim.hpp"
#include "wq_gemv_kernel.hpp"
#include "wq_mfma.hpp"
#include "wq_step_shared.hpp"

namespace wq {

constexpr int kMtPassChunks = 8;      // 16-byte chunks of a row per pass (128 inputs)
constexpr int kMtTileLds = 16 * 128;  // LDS bytes of one tile-pass

template <int U>
struct MtPassBuf {
  // one lane per row of the batch holds that row's scale
  static_assert(16 * U <= kWave, "at most 4 tiles per batch");
  u32x4 w[U][2];   // codes: tile u, rows (lane / 8) + 8 j, bytes 16 (lane % 8) .. + 15 of the pass
  u32x4 x[4];      // B operands of the pass's four MFMAs
  uint32_t sb;     // bf16 bits of the scale of row 16 U batch + lane (lanes < 16 U; clamped)
};

// bf16 pairs of the 8 codes in words d0, d1 (code 2i in the low half of pair i)
__device__ __forceinline__ void i8_to_bf16x8(uint32_t d0, uint32_t d1, uint32_t (&p)[4]) {
  const uint32_t d[2] = {d0, d1};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t f0 = __float_as_uint((float)(int8_t)(d[i]));
    const uint32_t f1 = __float_as_uint((float)(int8_t)(d[i] >> 8));
    const uint32_t f2 = __float_as_uint((float)(int8_t)(d[i] >> 16));
    const uint32_t f3 = __float_as_uint((float)(int8_t)(d[i] >> 24));
    p[2 * i] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);       // (upper half of f0, upper half of f1)
    p[2 * i + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
  }
}

// Loads pass `pass` of batch `batch`.  The lanes of a wave read 8 different
// rows per instruction, so the codes go through one buffer resource over the
// whole matrix (n row_bytes < 2^32, checked on the host) with per-lane
// offsets; rows past n and chunks past the row take an offset past the
// resource and read zero, as do tokens past M and inputs past k in the
// activations' resource.  With !ok every load reads zeros (empty resources)
// without touching memory, so a prefetch past the segment is issued like any
// other.
template <int M, int U>
__device__ __forceinline__ void mt_load_pass(const GemvArgs& a, int64_t batch, int pass, int lane, MtPassBuf<U>& bt,
                                             bool ok) {
  constexpr uint32_t kPast = 0xFFFFFFF0u;
  const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(a.w, ok ? (uint32_t)(a.n * a.row_bytes) : 0u);
  const int c = pass * kMtPassChunks + (lane & 7);   // this lane's chunk of the row
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t r = (batch * U + u) * 16 + 8 * j + (lane >> 3);
      const bool in = r < a.n && c < a.chunks;
      bt.w[u][j] = buffer_load16_nt(rw, in ? (uint32_t)(r * a.row_bytes) + (uint32_t)c * 16u : kPast);
    }
  }
  // B of MFMA m, lane 16 s + t: inputs pass 128 + 32 m + 8 s .. + 7 of token t
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(a.x, ok ? (uint32_t)(M * a.k * 2) : 0u);
  const uint32_t tok = (uint32_t)(lane & 15) * (uint32_t)(a.k * 2);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int64_t e = (int64_t)pass * 128 + 32 * m + 8 * (lane >> 4);
    bt.x[m] = buffer_load16(rx, e < a.k ? tok + (uint32_t)e * 2u : kPast);
  }
  int64_t rs = batch * U * 16 + (lane < 16 * U ? lane : 0);
  if (rs >= a.n) rs = a.n - 1;
  bt.sb = (uint32_t)*gmem(a.scale + rs);
}

// Accumulates one pass of U tiles into acc, through the wave's LDS tile
// `lds` (kMtTileLds bytes, reused for each tile: the wave's LDS accesses
// complete in order).
template <int U>
__device__ __forceinline__ void mt_accumulate(const MtPassBuf<U>& bt, f32x4 (&acc)[U], uint8_t* lds, int lane) {
  const int wr = lane >> 3, ws = lane & 7;          // stored row (+ 8 j) and 16-byte slot
  const int rr = lane & 15, rs = lane >> 4;         // A row and k-slot read back
  uint8_t* st0 = lds + wr * 128 + ((ws ^ ((wr >> 1) & 7)) << 4);               // row wr
  uint8_t* st1 = lds + (wr + 8) * 128 + ((ws ^ (((wr + 8) >> 1) & 7)) << 4);   // row wr + 8
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // Lanes read what other lanes stored: the wave's LDS accesses execute in
    // program order, and the wave barriers keep the compiler from moving
    // the reads above these stores or the next tile's stores above them.
    __builtin_amdgcn_wave_barrier();
    *reinterpret_cast<u32x4*>(st0) = bt.w[u][0];
    *reinterpret_cast<u32x4*>(st1) = bt.w[u][1];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // bytes 32 m + 8 s of row rr: slot 2 m + s / 2, half s % 2
      const uint2 v = *reinterpret_cast<const uint2*>(lds + rr * 128 +
                                                      (((2 * m + (rs >> 1)) ^ ((rr >> 1) & 7)) << 4) + ((rs & 1) << 3));
      uint32_t av[4];
      i8_to_bf16x8(v.x, v.y, av);
      const uint32_t b[4] = {bt.x[m][0], bt.x[m][1], bt.x[m][2], bt.x[m][3]};
      acc[u] = mfma_bf16(av, b, acc[u]);
    }
  }
}

// Scales and stores the 16 U rows x M tokens of batch `batch` (lane l holds
// rows 4 (l / 16) + r of each tile for token l % 16; `sb` is the scale of
// row 16 U batch + lane in lanes < 16 U).  Every lane must call it.
template <int M, int U>
__device__ __forceinline__ void mt_store(const GemvArgs& a, int64_t batch, int lane, const f32x4 (&acc)[U],
                                         uint32_t sb) {
  const int t = lane & 15, slot = lane >> 4;
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // the scale of this lane's row r sits in lane 16 u + 4 slot + r
      const uint32_t sbits = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * u + 4 * slot + r) * 4, (int)sb);
      const int64_t row = (batch * U + u) * 16 + 4 * slot + r;
      if (t < M && row < a.n) {
        const float v = acc[u][r] * __uint_as_float(sbits << 16);
        if (a.y32) *gmem(a.y32 + (int64_t)t * a.n + row) = v;
        if (a.y16) *gmem(a.y16 + (int64_t)t * a.n + row) = f32_to_bf16(v);
      }
    }
  }
}

// Accumulates one pass; after the batch's last pass, stores the batch and
// clears the accumulators.
template <int M, int U>
__device__ __forceinline__ void mt_finish_pass(const GemvArgs& a, int64_t batch, int pass, int passes, int lane,
                                               const MtPassBuf<U>& bt, f32x4 (&acc)[U], uint8_t* lds) {
  mt_accumulate<U>(bt, acc, lds, lane);
  if (pass + 1 < passes) return;
  mt_store<M, U>(a, batch, lane, acc, bt.sb);
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// The waves' share of one matrix segment: batches [lb, le) of `a`, claimed
// one at a time from `ctr` (zeroed by the caller).  Two pass buffers
// alternate, so the next pass's request is always in flight while one is
// consumed (the same discipline as the one-token kernel's stream_segment).
template <int M, int U>
__device__ __forceinline__ void mt_stream_segment(const GemvArgs& a, int64_t lb, int64_t le, int* ctr, int lane,
                                                  uint8_t* lds) {
  const int passes = a.cpl;
  int64_t cur = lb + claim_batch(ctr, lane);
  if (cur >= le) return;
  int64_t nxt = lb + claim_batch(ctr, lane);
  int pass = 0;
  f32x4 acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  MtPassBuf<U> A, B;
  mt_load_pass<M, U>(a, cur, 0, lane, A, true);
  for (;;) {
    int64_t c2 = cur;
    int p2 = pass + 1;
    if (p2 == passes) {
      c2 = nxt;
      p2 = 0;
    }
    bool more = c2 < le;
    mt_load_pass<M, U>(a, c2, p2, lane, B, more);
    if (more && p2 == 0) nxt = lb + claim_batch(ctr, lane);
    mt_finish_pass<M, U>(a, cur, pass, passes, lane, A, acc, lds);
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
    mt_load_pass<M, U>(a, c2, p2, lane, A, more);
    if (more && p2 == 0) nxt = lb + claim_batch(ctr, lane);
    mt_finish_pass<M, U>(a, cur, pass, passes, lane, B, acc, lds);
    if (!more) {
      wait_vmem_all();
      break;
    }
    cur = c2;
    pass = p2;
  }
}

// mats: per-matrix descriptors (batch = U tiles of 16 rows; `cpl` holds the
// number of passes per row); ranges and balance as in the one-token step.
template <int M, int U, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemm_i8_step_kernel(const GemvArgs* __restrict__ mats, StepCuts cuts) {
  __shared__ __attribute__((aligned(16))) uint8_t tiles[WAVES][kMtTileLds];
  __shared__ int ctr;
  const int lane = lane_id();
  uint8_t* lds = tiles[threadIdx.x >> 6];
  step_frame<WAVES>(mats, cuts, [&](const GemvArgs& a, int64_t lb, int64_t le) {
    __syncthreads();   // every wave has left the previous segment
    if (threadIdx.x == 0) ctr = 0;
    __syncthreads();
    mt_stream_segment<M, U>(a, lb, le, &ctr, lane, lds);
  });
}

// One matrix (wq_gemm_smallM_int8): workgroup b takes batches b, b + grid,
// ... of U 16-row tiles (one activation load serves the U tiles); its waves
// split the batch's passes (wave w: passes w, w + WAVES, ...), and their sums
// meet in LDS, added in wave order, so results do not depend on timing.
template <int M, int U, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemm_i8_smallm_kernel(GemvArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tiles[WAVES][kMtTileLds];
  __shared__ f32x4 red[WAVES][U][kWave];
  const int lane = lane_id();
  const int wave = (int)(threadIdx.x >> 6);
  uint8_t* lds = tiles[wave];
  const int passes = a.cpl;
  for (int64_t batch = blockIdx.x; batch < a.batches; batch += gridDim.x) {
    f32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    MtPassBuf<U> A, B;
    int p = wave;
    mt_load_pass<M, U>(a, batch, p, lane, A, p < passes);
    for (;;) {
      p += WAVES;
      bool more = p < passes;
      mt_load_pass<M, U>(a, batch, p, lane, B, more);
      mt_accumulate<U>(A, acc, lds, lane);
      if (!more) {
        wait_vmem_all();
        break;
      }
      p += WAVES;
      more = p < passes;
      mt_load_pass<M, U>(a, batch, p, lane, A, more);
      mt_accumulate<U>(B, acc, lds, lane);
      if (!more) {
        wait_vmem_all();
        break;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) red[wave][u][lane] = acc[u];
    __syncthreads();
    if (wave == 0) {
      f32x4 tot[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        tot[u] = red[0][u][lane];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) tot[u] += red[w][u][lane];
      }
      int64_t rs = batch * 16 * U + (lane < 16 * U ? lane : 0);
      if (rs >= a.n) rs = a.n - 1;
      mt_store<M, U>(a, batch, lane, tot, (uint32_t)*gmem(a.scale + rs));
    }
    __syncthreads();
  }
}

// One large matrix (wq_gemm_smallM_int8) in the claiming frame of
// wq_claim.hpp: a block is a batch of U 16-row tiles, a unit kMtUnitPasses
// passes (1024 inputs) of its rows.  A wave streams its units' passes with
// two buffers alternating, the next unit's first pass requested while the
// current unit's last one is reduced.  A unit's sums (the lanes of tokens
// < M: four rows each per tile) go to its LDS slot; the block's last unit
// adds the slots in unit order, scales and stores the rows.
constexpr int kMtUnitPasses = 8;
constexpr int kMtMaxUnits = 32;   // rows of up to 32768 inputs

template <int M, int U, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemm_i8_matrix_kernel(GemvArgs a, MatrixClaim* claim, int32_t cap) {
  constexpr int R = 2;
  __shared__ __attribute__((aligned(16))) uint8_t tiles[WAVES][kMtTileLds];
  __shared__ f32x4 part[R][kMtMaxUnits][U][4][M];   // slot, unit, tile, lane / 16, token
  __shared__ MatrixUnitLds<R> ul;
  const int lane = lane_id();
  const int wave = (int)(threadIdx.x >> 6);
  const int t = lane & 15, rq = lane >> 4;
  uint8_t* lds = tiles[wave];
  const int passes = a.cpl;
  const int ups = (passes + kMtUnitPasses - 1) / kMtUnitPasses;   // units per block (1..kMtMaxUnits)
  const int first = ups < WAVES ? ups : WAVES;
  MatrixUnits<R> mu{ul, claim, ups, cap, (int)a.batches, lane};
  mu.init(wave, first);
  __syncthreads();

  int jl = 0, u = wave, gb = (int)blockIdx.x;
  bool have = wave < first;
  if (!have) have = mu.claim_next(jl, u, gb);
  if (!have) {
    mu.end_launch();
    return;
  }
  f32x4 acc[U];
#pragma unroll
  for (int i = 0; i < U; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  int p = u * kMtUnitPasses;                                       // pass in A (then B, ...)
  int pe = p + kMtUnitPasses < passes ? p + kMtUnitPasses : passes;
  int jn = 0, un = 0, gn = 0;
  bool more = mu.claim_next(jn, un, gn);                            // the unit after this one
  MtPassBuf<U> A, B;
  mt_load_pass<M, U>(a, gb, p, lane, A, true);

  // consumes the pass in `cur` after requesting its successor into `nx`;
  // false once the wave has no more work
  auto step = [&](const MtPassBuf<U>& cur, MtPassBuf<U>& nx) -> bool {
    const bool same = p + 1 < pe;
    mt_load_pass<M, U>(a, same ? gb : gn, same ? p + 1 : un * kMtUnitPasses, lane, nx, same || more);
    mt_accumulate<U>(cur, acc, lds, lane);
    if (same) {
      ++p;
      return true;
    }
    // the unit is done: its sums into its slot, once the slot's previous
    // block is out
    const int sl = jl % R;
    mu.wait_slot(jl);
    if (t < M) {
#pragma unroll
      for (int i = 0; i < U; ++i) part[sl][u][i][rq][t < M ? t : 0] = acc[i];
    }
#pragma unroll
    for (int i = 0; i < U; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (mu.unit_done(jl)) {
      // the block's last unit: add its units' sums in order, scale, store
      f32x4 tot[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        tot[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (t < M) {
          tot[i] = part[sl][0][i][rq][t < M ? t : 0];
          for (int w = 1; w < ups; ++w) tot[i] += part[sl][w][i][rq][t < M ? t : 0];
        }
      }
      int64_t rs = (int64_t)gb * 16 * U + (lane < 16 * U ? lane : 0);
      if (rs >= a.n) rs = a.n - 1;
      mt_store<M, U>(a, gb, lane, tot, (uint32_t)*gmem(a.scale + rs));
      mu.release(jl);
    }
    if (!more) return false;
    jl = jn;
    u = un;
    gb = gn;
    p = u * kMtUnitPasses;
    pe = p + kMtUnitPasses < passes ? p + kMtUnitPasses : passes;
    more = mu.claim_next(jn, un, gn);
    return true;
  };
  // the prefetch left in flight is drained on the way out
  for (;;) {
    if (!step(A, B)) break;
    if (!step(B, A)) break;
  }
  wait_vmem_all();
  mu.end_launch();
}

}  // namespace wq
