// Speculative-verify product (int4 G=32 weights, 2 <= M <= 8 token rows) on
// the matrix cores: v_mfma_f32_16x16x32_bf16.
//
// One MFMA multiplies a 16 x 32 A tile by a 32 x 16 B tile.  Here a "quad"
// is 16 weight rows x 4 consecutive groups (128 inputs):
//   * A: lane l holds 8 k-values of row (l % 16) in k-slot (l / 16); the quad
//     is decoded so that lane l's 16 loaded bytes -- group (l / 16) of its row
//     -- feed k-slot (l / 16) of four MFMAs (word j of the chunk -> MFMA j).
//     Codes become exact bf16 (128 + q) as in the VALU path.
//   * B is block diagonal: output column c = 4 * slot + token (tokens 0..3 in
//     the first column set, 4..7 in the second), and lane (slot q', column c)
//     holds that token's activations of group q' only when c belongs to slot
//     q'; every other B element is zero.  So D[row][c] is the sum over ONE
//     group, and the group's scale and zero are applied exactly afterwards:
//     y += s * D + (z - 128 s) * (sum of the group's activations).
//   * D: lane l holds rows 4 * (l / 16) + r (r < 4) of column l % 16.
// Activations are staged in LDS per K-window (pre-permuted bf16 pairs and
// per-group sums; once per matrix when a window holds all of K).  The waves of
// a workgroup take the window's work items in turn for the workgroup's block
// of 16 * RT rows, and their totals meet in LDS in a fixed order at the end
// of the block.  No atomics: results are bitwise reproducible.
#pragma once

#include <stdint.h>

#include "wq_formats.hpp"

namespace wq {

// The configuration used by both entry points (chosen by timing the
// Llama-3.1-70B verify shapes at 3..8 tokens): blocks of 2 row tiles (32
// rows), K windows of 256 groups, 12 waves, one item prefetched, items of 2
// quads (32 contiguous code bytes per lane).
constexpr int kMfmaRT = 2, kMfmaKW = 256, kMfmaWaves = 12, kMfmaPF = 1, kMfmaOct = 2;
constexpr int kMfmaMaxK = 131072;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct MfmaArgs {
  const uint16_t* x;     // [m][k] bf16
  const uint8_t* w;      // [n][k/2]
  const uint32_t* sz;    // [n][words]: group c >> gshift of 32-input chunk c
  float* y32;            // [m][n] or null
  uint16_t* y16;         // [m][n] or null
  int64_t n;
  int64_t k;
  int64_t blocks;        // ceil(n / (16 * RT))
  int32_t groups;        // k / 32 (32-input chunks)
  int32_t gshift;        // log2(G / 32) for groups of G inputs; a per-row group's shift exceeds any chunk index
  int64_t words;         // (scale, zero) words per row
};

template <int M, int RT, int KW, int WAVES>
struct alignas(16) MfmaShared {
  static constexpr int kSets = (M + 3) / 4;
  // permuted activation pairs per (token, group); each token's row is padded
  // by 16 bytes so the four tokens read by one k-slot sit in different banks
  static constexpr int kRow = KW * 16 + 4;
  uint32_t xs[M][kRow];
  float gs[M][KW + 1];                      // per-group activation sums; rows padded so the
                                            // tokens one lane quad reads sit in different banks
  alignas(16) uint32_t zero[16];            // B operand of columns outside a slot
  float red[WAVES][RT][kSets][4][16];       // per-wave totals (lanes with column < 4)
};

__device__ __forceinline__ f32x4 mfma_bf16(const uint32_t (&a)[4], const uint32_t (&b)[4], f32x4 c) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  u4 av = {a[0], a[1], a[2], a[3]};
  u4 bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), c,
                                                 0, 0, 0);
}

// Byte offset of 16-byte slot `slot` of row `row` in a 16-row x 128-byte
// LDS tile: slots XOR-swizzled by row pair, so 16 lanes storing two rows of
// 8 slots, or reading one slot of 16 rows, touch distinct banks.
__device__ __forceinline__ int mfma_tile_at(int row, int slot) { return row * 128 + ((slot ^ ((row >> 1) & 7)) << 4); }

template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Activations of groups [g0, g0 + kw) for all M tokens, staged into LDS in
// two phases: issue() requests this thread's pieces (token, group) -- all
// of them at once, through a buffer resource over the M token rows -- and
// finish() writes them in the layout above.  Issued before a workgroup's
// first weights, they arrive first, and their wait does not hold for the
// weight loads behind them.
template <int M, int RT, int KW, int WAVES>
struct MfmaStage {
  static constexpr int kPieces = (M * KW + WAVES * 64 - 1) / (WAVES * 64);
  u32x4 v[kPieces][4];

  __device__ __forceinline__ void issue(const MfmaArgs& a, int g0, int kw) {
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(a.x, (uint32_t)(M * a.k * 2));
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
      const int it = (int)threadIdx.x + q * WAVES * 64;
      const int t = it / kw, g = it - (it / kw) * kw;
      const uint32_t off = t < M ? (uint32_t)t * (uint32_t)(a.k * 2) + (uint32_t)(g0 + g) * 64u : 0x80000000u;
#pragma unroll
      for (int h = 0; h < 4; ++h) v[q][h] = buffer_load16(rx, off + 16u * h);
    }
  }
  // One piece at a time instead (fewer registers), for a restaging inside
  // the block loop where all of them in flight would spill.
  __device__ static __forceinline__ void serial(const MfmaArgs& a, int g0, int kw, MfmaShared<M, RT, KW, WAVES>& sh) {
    for (int it = threadIdx.x; it < M * kw; it += WAVES * 64) {
      const int t = it / kw;
      const int g = it - t * kw;
      const FmtInt4::X xv = FmtInt4::load_x(a.x + (int64_t)t * a.k, g0 + g, true);
#pragma unroll
      for (int i = 0; i < 16; ++i) sh.xs[t][16 * g + i] = xv.p[i];
      sh.gs[t][g] = xv.gsum;
    }
  }
  __device__ __forceinline__ void finish(MfmaShared<M, RT, KW, WAVES>& sh, int kw) const {
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
      const int it = (int)threadIdx.x + q * WAVES * 64;
      const int t = it / kw, g = it - (it / kw) * kw;
      if (t < M) {
        const FmtInt4::X xv = FmtInt4::from_words(v[q]);
#pragma unroll
        for (int i = 0; i < 16; ++i) sh.xs[t][16 * g + i] = xv.p[i];
        sh.gs[t][g] = xv.gsum;
      }
    }
  }
};

// One work item: OCT quads of a block's RT row tiles.  Lane (rq, col) loads
// the 16 * OCT contiguous code bytes of groups gb + OCT rq + o (o < OCT) of
// row col, so quad o is made of groups gb + OCT rq' + o over the four k-slots;
// and for each quad the (scale, zero) words of its D rows 4 rq + r for the
// group of its D column, gb + OCT slot + o.  Rows past n and groups past k/32
// read as zero.
template <int RT, int OCT>
struct ItemData {
  u32x4 w[RT][OCT];
  uint32_t sz[RT][OCT][4];
};

// LT (line-wide, OCT = 2): the item's codes are read as two loads of 8 rows
// x 128 bytes per tile (lane l: row l / 8 (+ 8), group gb + l % 8) and reach
// the layout above through a per-wave LDS tile (mfma_blocks).
// With !any every load reads zero (empty resources) without touching memory,
// so a conditional request is issued like any other.
template <int RT, int OCT, bool LT>
__device__ __forceinline__ void load_item(const MfmaArgs& a, int64_t n0, int64_t gb, int rq, int col, int slot,
                                          ItemData<RT, OCT>& q, bool any = true) {
  static_assert(!LT || OCT == 2, "a line-wide item is 8 groups of 16 rows");
  const int lane = 16 * rq + col;
  const uint32_t row_bytes = (uint32_t)(a.k / 2);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t rbase = n0 + 16 * rt;
    const int64_t rows_left = any ? a.n - rbase : 0;
    const uint32_t rows_ok = rows_left <= 0 ? 0u : (rows_left >= 16 ? 16u : (uint32_t)rows_left);
    const int64_t rb = rows_left > 0 ? rbase : 0;
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(a.w + rb * (a.k / 2), rows_ok * row_bytes);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.sz + rb * a.words, rows_ok * (uint32_t)a.words * 4u);
#pragma unroll
    for (int o = 0; o < OCT; ++o) {
      const int64_t g = LT ? gb + (lane & 7) : gb + OCT * rq + o;
      const uint32_t row = LT ? (uint32_t)(8 * o + (lane >> 3)) : (uint32_t)col;
      q.w[rt][o] = buffer_load16_nt(rw, g < a.groups ? row * row_bytes + (uint32_t)g * 16u : 0x80000000u);
    }
#pragma unroll
    for (int o = 0; o < OCT; ++o) {
      const int64_t ge = gb + OCT * slot + o;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t offs = ge < a.groups
                                  ? ((uint32_t)(4 * rq + r) * (uint32_t)a.words + (uint32_t)(ge >> a.gshift)) * 4u
                                  : 0x80000000u;
        q.sz[rt][o][r] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)offs, 0, 0);
      }
    }
  }
}

// Next item of this wave's sequence (block, window start, item) after the
// given one: items wave, wave + WAVES, ... of each window, windows in order,
// then the next block of the range.  False when the wave has no more work.
template <int KW, int WAVES, int OCT>
__device__ __forceinline__ bool next_item(const MfmaArgs& a, int64_t b_end, int64_t b_step, int wave, int64_t& blk,
                                          int& g0, int& it) {
  it += WAVES;
  for (;;) {
    const int kw = (a.groups - g0) < KW ? (a.groups - g0) : KW;
    if (4 * OCT * it < kw) return true;
    g0 += KW;
    it = wave;
    if (g0 >= a.groups) {
      g0 = 0;
      blk += b_step;
      if (blk >= b_end) return false;
    }
  }
}

// One workgroup's share of a matrix: blocks b_first, b_first + b_step, ...
// below b_end, each of 16 * RT rows.  The block's K range is walked in
// windows of KW groups whose activations are staged in LDS (once per call
// when one window holds all of K), and the WAVES waves take the window's
// items in turn.  PF = 1 keeps the next item's loads in flight while one
// computes.  Every thread of the workgroup must make the same call.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  return reinterpret_cast<T*>(uniform64(reinterpret_cast<int64_t>(p)));
}

// A descriptor whose fields the compiler can keep in scalar registers: the
// buffer resources built from them must be wave-uniform, or every buffer
// load turns into a loop over the distinct values.
__device__ __forceinline__ MfmaArgs uniform_args(const MfmaArgs& a) {
  MfmaArgs u;
  u.x = uniform_ptr(a.x);
  u.w = uniform_ptr(a.w);
  u.sz = uniform_ptr(a.sz);
  u.y32 = uniform_ptr(a.y32);
  u.y16 = uniform_ptr(a.y16);
  u.n = uniform64(a.n);
  u.k = uniform64(a.k);
  u.blocks = uniform64(a.blocks);
  u.groups = __builtin_amdgcn_readfirstlane(a.groups);
  u.gshift = __builtin_amdgcn_readfirstlane(a.gshift);
  u.words = uniform64(a.words);
  return u;
}

template <int M, int RT, int KW, int WAVES, int PF, int OCT, bool LT>
__device__ __forceinline__ void mfma_blocks(const MfmaArgs& a_in, int64_t b_first, int64_t b_end, int64_t b_step,
                                            MfmaShared<M, RT, KW, WAVES>& sh, uint8_t* tile) {
  constexpr int SETS = (M + 3) / 4;
  const MfmaArgs a = uniform_args(a_in);
  b_first = uniform64(b_first);
  b_end = uniform64(b_end);
  b_step = uniform64(b_step);
  const int lane = lane_id();
  const int wave = wave_id();
  const int rq = lane >> 4;          // k-slot of A, row quarter of D
  const int col = lane & 15;         // row of A, column of D
  const int slot = col >> 2;         // group slot of this D column
  const int tok0 = col & 3;          // token of this D column in set 0
  const FmtInt4::K kc = FmtInt4::consts();
  const bool single = a.groups <= KW;   // one window: stage it once

  ItemData<RT, OCT> nxt;
  int64_t pblk = b_first;
  int pg0 = 0, pit = wave - WAVES;
  bool pending = false;
  // the first window's activations are requested before the first item and
  // staged before the loop
  const int kw0 = a.groups < KW ? a.groups : KW;
  {
    MfmaStage<M, RT, KW, WAVES> stage;
    stage.issue(a, 0, kw0);
    __builtin_amdgcn_sched_barrier(0);
    // requested on every path (empty when there is none), so the staging's
    // wait below holds only for the activations issued before it
    if (PF) {
      pending = pblk < b_end && next_item<KW, WAVES, OCT>(a, b_end, b_step, wave, pblk, pg0, pit);
      load_item<RT, OCT, LT>(a, pending ? pblk * 16 * RT : 0, pending ? (int64_t)pg0 + 4 * OCT * pit : 0, rq, col,
                             slot, nxt, pending);
    }
    stage.finish(sh, kw0);
  }
  __syncthreads();
  bool first_window = true;           // the first block's first window is staged
  uint32_t bop[SETS][4][4];          // B operands of the current quad (see below)
#pragma unroll
  for (int st = 0; st < SETS; ++st)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) bop[st][j][e] = 0u;

  for (int64_t blk = b_first; blk < b_end; blk += b_step) {
    const int64_t n0 = blk * 16 * RT;
    float tot[RT][SETS][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int s = 0; s < SETS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[rt][s][r] = 0.0f;

    for (int g0 = 0; g0 < a.groups; g0 += KW) {
      const int kw = (a.groups - g0) < KW ? (a.groups - g0) : KW;
      if (!single && !first_window) {
        __syncthreads();                     // previous window fully consumed
        if constexpr (MfmaStage<M, RT, KW, WAVES>::kPieces <= 2) {
          MfmaStage<M, RT, KW, WAVES> stage;
          stage.issue(a, g0, kw);
          stage.finish(sh, kw);
        } else {
          MfmaStage<M, RT, KW, WAVES>::serial(a, g0, kw, sh);
        }
        __syncthreads();
      }
      first_window = false;
      const int items = (kw + 4 * OCT - 1) / (4 * OCT);
      for (int it = wave; it < items; it += WAVES) {
        const int64_t gb = g0 + 4 * OCT * it;
        ItemData<RT, OCT> cur;
        if (PF) {
          cur = nxt;
          pending = next_item<KW, WAVES, OCT>(a, b_end, b_step, wave, pblk, pg0, pit);
          if (pending) load_item<RT, OCT, LT>(a, pblk * 16 * RT, (int64_t)pg0 + 4 * OCT * pit, rq, col, slot, nxt);
        } else {
          load_item<RT, OCT, LT>(a, n0, gb, rq, col, slot, cur);
        }
        // LT: each tile's 16 rows x 8 groups pass through the wave's LDS
        // tile (slots XOR-swizzled by row pair; the wave's LDS accesses
        // complete in order, so the next tile's stores follow these reads);
        // lane (rq, col) reads back groups OCT rq + o of row col
        u32x4 wl[RT][OCT];
        if constexpr (LT) {
          const int lane = 16 * rq + col, wr = lane >> 3, ws = lane & 7;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            // lanes read what other lanes stored: the wave barriers keep the
            // compiler from reordering these LDS accesses across lanes' roles
            __builtin_amdgcn_wave_barrier();
            *reinterpret_cast<u32x4*>(tile + mfma_tile_at(wr, ws)) = cur.w[rt][0];
            *reinterpret_cast<u32x4*>(tile + mfma_tile_at(wr + 8, ws)) = cur.w[rt][1];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int o = 0; o < OCT; ++o) wl[rt][o] = *reinterpret_cast<const u32x4*>(tile + mfma_tile_at(col, OCT * rq + o));
          }
        }
#pragma unroll
        for (int o = 0; o < OCT; ++o) {
          // B operands of quad o.  Only the lanes whose column slot equals
          // their k-slot (and whose token exists) ever hold data: the others
          // keep the zeros they started with, so they read no LDS at all.
          float xsum[SETS];
          const int gl = 4 * OCT * it + OCT * rq + o;     // this lane's B group (window-local)
          const int ge = 4 * OCT * it + OCT * slot + o;   // the group of this lane's D column
#pragma unroll
          for (int s = 0; s < SETS; ++s) {
            const int t = 4 * s + tok0;
            if (slot == rq && t < M) {
              const uint32_t* src = gl < kw ? &sh.xs[t][16 * gl] : &sh.zero[0];
#pragma unroll
              for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) bop[s][j][e] = src[4 * j + e];
            }
            xsum[s] = (t < M && ge < kw) ? sh.gs[t < M ? t : 0][ge < kw ? ge : 0] : 0.0f;
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            FmtInt4::D d;
            FmtInt4::decode(LT ? wl[rt][o] : cur.w[rt][o], d, kc);
#pragma unroll
            for (int s = 0; s < SETS; ++s) {
              f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const uint32_t av[4] = {d.t[4 * j], d.t[4 * j + 1], d.t[4 * j + 2], d.t[4 * j + 3]};
                acc = mfma_bf16(av, bop[s][j], acc);
              }
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float sc = __uint_as_float(cur.sz[rt][o][r] << 16);
                const float zc = __uint_as_float(cur.sz[rt][o][r] & 0xFFFF0000u);
                float v = fmaf(sc, acc[r], tot[rt][s][r]);
                tot[rt][s][r] = fmaf(fmaf(-128.0f, sc, zc), xsum[s], v);
              }
            }
          }
        }
      }
    }

    // sum the four group slots of each token (columns c, c+4, c+8, c+12 of a
    // 16-lane row), then the waves in a fixed order, then store
    if (single) __syncthreads();             // the previous block's totals are read
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int s = 0; s < SETS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = tot[rt][s][r];
          v += dpp_row<0x124>(v);     // row_ror:4
          v += dpp_row<0x128>(v);     // row_ror:8
          if (col < 4) sh.red[wave][rt][s][r][4 * rq + col] = v;
        }
    __syncthreads();
    for (int i = threadIdx.x; i < RT * SETS * 4 * 16; i += WAVES * 64) {
      const int c16 = i & 15;
      const int r = (i >> 4) & 3;
      const int s = (i >> 6) % SETS;
      const int rt = (i >> 6) / SETS;
      const int t = 4 * s + (c16 & 3);
      const int64_t row = n0 + 16 * rt + 4 * (c16 >> 2) + r;
      if (t < M && row < a.n) {
        float v = sh.red[0][rt][s][r][c16];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) v += sh.red[w][rt][s][r][c16];
        if (a.y32) *gmem(a.y32 + ((int64_t)t * a.n + row)) = v;
        if (a.y16) *gmem(a.y16 + ((int64_t)t * a.n + row)) = f32_to_bf16(v);
      }
    }
  }
}

// One matrix: workgroups take blocks blockIdx.x, blockIdx.x + gridDim.x, ...
// LT: line-wide code loads through a 2 KiB LDS tile per wave (fits beside
// the activation window up to 7 tokens).
template <int M, int RT, int KW, int WAVES, int PF, int OCT, bool LT>
__global__ __launch_bounds__(WAVES * 64) void gemm_mfma_kernel(MfmaArgs a) {
  __shared__ MfmaShared<M, RT, KW, WAVES> sh;
  __shared__ __attribute__((aligned(16))) uint8_t tiles[LT ? WAVES : 1][LT ? 16 * 128 : 16];
  if (threadIdx.x < 16) sh.zero[threadIdx.x] = 0u;
  mfma_blocks<M, RT, KW, WAVES, PF, OCT, LT>(a, blockIdx.x, a.blocks, gridDim.x, sh, tiles[LT ? threadIdx.x >> 6 : 0]);
}

}  // namespace wq
