// Several token rows (2 <= M <= 8) against int4 G=32 weights on the matrix
// cores: the speculative-verify product of a decode step, one persistent
// launch per step.
//
// One v_mfma_f32_16x16x32_bf16 computes D = A B + C for a 16 x 32 A and a
// 32 x 16 B.  Here B holds WEIGHTS and A holds ACTIVATIONS:
//   * B: lane l (k-slot l / 16, column l % 16) decodes the 16 code bytes it
//     loaded -- one group of weight row (l % 16) of the tile -- into exact bf16
//     values 128 + q (the nibble-into-mantissa decode of the VALU path); word
//     j of the chunk feeds MFMA j, so four MFMAs cover the 32 weights.  The
//     four k-slots hold four different groups of the 16 rows (a "quad").
//   * A is block diagonal: row 4 * slot + t is token t (of a set of four)
//     restricted to the group of k-slot `slot`; every other element is zero.
//     Only lanes 20 s + t (s, t < 4) carry data, read from LDS; the other
//     lanes hold zeros and read nothing.
//   * So D[4 * slot + t][n] is token t's dot product with ONE group of row n,
//     and lane l holds D rows 4 (l / 16) + r, column l % 16: the four tokens'
//     sums for exactly the (row, group) whose codes and (scale, zero) word it
//     loaded itself.  The group's scale and zero are applied exactly:
//     y_t += s * D + (z - 128 s) * (sum of the group's activations of t).
// Tokens 4..7 use a second set of MFMAs (same B, second A).
//
// Work decomposition: one workgroup per CU owns a contiguous range of the
// step's blocks of RT 16-row tiles (equal weight bytes per workgroup, cut on
// the host); a wave's A operands serve all RT tiles of its block.
// Per matrix segment the activations of all M tokens are staged in LDS in
// windows of KW groups (pre-permuted bf16 pairs + per-group sums).  When one
// window holds the whole row (k <= 32 KW) it is staged once and the waves
// claim tiles from an LDS counter, each streaming whole rows; longer rows
// walk the windows in rounds of one tile per wave, with a barrier per
// window.  Each lane accumulates its slot's groups, the four slots are summed
// with cross-lane swaps in a fixed order and the totals stored: results are
// bitwise reproducible whichever wave takes a tile.
#pragma once

#include <stdint.h>

#include "wq_formats.hpp"
#include "wq_step_shared.hpp"

namespace wq {

// Longest row (inputs) the verify kernel accepts (offsets stay in 32 bits).
constexpr int kVerifyMaxK = 131072;

typedef __bf16 vbf16x8 __attribute__((ext_vector_type(8)));
typedef float vf32x4 __attribute__((ext_vector_type(4)));

// Activations of one K window for up to M tokens.  Token rows are padded by
// 16 bytes so the four tokens one k-slot reads sit in different banks.
template <int M, int KW>
struct alignas(16) VerifyShared {
  static constexpr int kSets = (M + 3) / 4;
  static constexpr int kRow = KW * 16 + 4;
  uint32_t xs[M][kRow];          // pre-permuted bf16 pairs, 16 words per group
  float gs[KW][kSets][4];        // per-group activation sums, [group][set][token in set]
};

template <int RT, int OCT>
struct VerifyItem {
  u32x4 w[RT][OCT];      // codes of OCT consecutive groups of one row of each of RT tiles
};

// (scale, zero) words of the 16 rows of each tile for a window of kSzWin
// groups, loaded with full cache lines (8 rows x 32 groups per wave-wide
// load) and passed through a per-wave LDS buffer, from which each lane reads
// the words of its own (row, group).  Loads whose lanes span 16 rows touch a
// line per row for a few bytes each; the address path, not HBM, then sets the
// pace.
constexpr int kSzWin = 32;
constexpr int kSzRow = kSzWin + 4;   // LDS words per row (16-byte aligned, skewed banks)

template <int RT>
struct SzWindow {
  u32x4 r[RT][2];   // rows 8h + lane / 8, groups 4 (lane % 8) .. + 3
};

__device__ __forceinline__ vf32x4 mfma16x16x32(const uint32_t (&a)[4], const uint32_t (&b)[4], vf32x4 c) {
  const u32x4 av = {a[0], a[1], a[2], a[3]};
  const u32x4 bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(vbf16x8, av), __builtin_bit_cast(vbf16x8, bv), c,
                                                 0, 0, 0);
}

// Stages groups [g0, g0 + kpad) of every token; groups at or past the row's
// end are zero.
template <int M, int KW, int THREADS>
__device__ __forceinline__ void verify_stage(const GemvArgs& a, int g0, int kpad, VerifyShared<M, KW>& sh) {
  constexpr int SETS = VerifyShared<M, KW>::kSets;
#pragma unroll 1
  for (int it = threadIdx.x; it < 4 * SETS * kpad; it += THREADS) {
    const int t = it / kpad;
    const int g = it - t * kpad;
    const int gg = g0 + g;
    if (t < M) {
      const FmtInt4::X xv = FmtInt4::load_x(a.x + (int64_t)t * a.k, gg, gg < a.chunks);
#pragma unroll
      for (int h = 0; h < 4; ++h)
        *reinterpret_cast<u32x4*>(&sh.xs[t][16 * g + 4 * h]) =
            u32x4{xv.p[4 * h], xv.p[4 * h + 1], xv.p[4 * h + 2], xv.p[4 * h + 3]};
      sh.gs[g][t >> 2][t & 3] = xv.gsum;
    } else {
      sh.gs[g][t >> 2][t & 3] = 0.0f;
    }
  }
}

// Loads the codes of item `it` of window [g0, ...) of block `blk` (tiles
// RT blk .. RT blk + RT - 1): OCT quads of 4 consecutive groups (k-slot s of
// quad o = group 4 o + s of the item) for the 16 rows of each tile.  With QL a wave-wide load is laid out so that each quad
// of lanes reads ONE row (lane (row = lane / 4, k-slot = lane % 4)) and
// verify_item moves each word to the MFMA lane (k-slot = lane / 16, row =
// lane % 16) with a cross-lane permute; without QL each lane loads its own
// MFMA chunk.  Rows past n and groups past the row read as zero, and so does
// everything with !any: the loads are issued on every path, so code after a
// conditional prefetch waits only for the item it consumes.
template <int RT, int OCT, bool QL>
__device__ __forceinline__ void verify_load(const GemvArgs& a, int64_t blk, int g0, int it, int lane,
                                            VerifyItem<RT, OCT>& q, bool any = true) {
  const uint32_t row_bytes = (uint32_t)a.row_bytes;
  const int lrow = QL ? lane >> 2 : lane & 15;
  const int gl = g0 + it * 4 * OCT + (QL ? lane & 3 : lane >> 4);   // this lane's group of quad 0
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t rbase = (blk * RT + rt) * 16;
    const int64_t left = a.n - rbase;
    // !any empties the (wave-uniform) resource rather than the per-lane
    // offsets, which keeps the loads free of branches
    const bool live = any && left > 0;
    const uint32_t rows_ok = !live ? 0u : (left >= 16 ? 16u : (uint32_t)left);
    const int64_t rb = live ? rbase : 0;
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(a.w + rb * a.row_bytes, rows_ok * row_bytes);
#pragma unroll
    for (int o = 0; o < OCT; ++o) {
      const bool ok = gl + 4 * o < a.chunks;
      q.w[rt][o] =
          buffer_load16_nt(rw, ok ? (uint32_t)lrow * row_bytes + (uint32_t)(gl + 4 * o) * 16u : 0x80000000u);
    }
  }
}

// Loads the (scale, zero) words of groups [gw, gw + kSzWin) of block `blk`
// (zeros with !any).
template <int RT>
__device__ __forceinline__ void sz_load(const GemvArgs& a, int64_t blk, int gw, int lane, SzWindow<RT>& z,
                                        bool any = true) {
  const int g = gw + 4 * (lane & 7);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t rbase = (blk * RT + rt) * 16;
    const int64_t left = a.n - rbase;
    const bool live = any && left > 0;
    const uint32_t rows_ok = !live ? 0u : (left >= 16 ? 16u : (uint32_t)left);
    const int64_t rb = live ? rbase : 0;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.sz + rb * a.chunks, rows_ok * (uint32_t)a.chunks * 4u);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t row = (uint32_t)(8 * h + (lane >> 3));
      z.r[rt][h] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     rs, g < a.chunks ? (int)((row * (uint32_t)a.chunks + (uint32_t)g) * 4u) : (int)0x80000000, 0, 2));
    }
  }
}

// Writes a loaded window into the wave's LDS buffer; words of groups past
// the row's end (which belong to the next row) become zero.
template <int RT>
__device__ __forceinline__ void sz_put(const GemvArgs& a, int gw, int lane, const SzWindow<RT>& z,
                                       uint32_t (*buf)[16][kSzRow]) {
  const int g = gw + 4 * (lane & 7);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 v = z.r[rt][h];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (g + e >= a.chunks) v[e] = 0u;
      *reinterpret_cast<u32x4*>(&buf[rt][8 * h + (lane >> 3)][4 * (lane & 7)]) = v;
    }
}

// Word `v` of lane 4 * col + rq, delivered to lane (rq, col) = 16 rq + col.
__device__ __forceinline__ uint32_t to_mfma_lane(uint32_t v, int src_addr) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src_addr, (int)v);
}

// A operands of lane (rq, col) for one quad: the activations of token
// 4 st + (col & 3) for group `ga` when the lane's A row belongs to its k-slot
// (col / 4 == rq) and the token exists.  Other lanes never write `av`, which
// keeps the zeros it was created with, so they touch no LDS.
template <int M, int KW>
__device__ __forceinline__ void verify_a(const VerifyShared<M, KW>& sh, int ga, int rq, int col,
                                         uint32_t (&av)[VerifyShared<M, KW>::kSets][4][4]) {
  constexpr int SETS = VerifyShared<M, KW>::kSets;
#pragma unroll
  for (int st = 0; st < SETS; ++st) {
    const int t = 4 * st + (col & 3);
    if ((col >> 2) == rq && t < M) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(&sh.xs[t < M ? t : 0][16 * ga + 4 * j]);
        av[st][j][0] = v[0];
        av[st][j][1] = v[1];
        av[st][j][2] = v[2];
        av[st][j][3] = v[3];
      }
    }
  }
}

// Accumulates one item into y[tile][set][token]; `il` is the item's first
// group within the staged activation window and `iz` within the (scale,
// zero) window held in `szb`.
template <int M, int KW, int RT, int OCT, bool QL, bool SB>
__device__ __forceinline__ void verify_item(const VerifyItem<RT, OCT>& q, int il, int iz, int rq, int col,
                                            const VerifyShared<M, KW>& sh, const uint32_t (*szb)[16][kSzRow],
                                            const FmtInt4::K& kc, uint32_t (&av)[VerifyShared<M, KW>::kSets][4][4],
                                            float (&y)[RT][VerifyShared<M, KW>::kSets][4]) {
  constexpr int SETS = VerifyShared<M, KW>::kSets;
  const int src = (4 * col + rq) * 4;   // byte address of the lane holding this lane's codes (QL)
#pragma unroll
  for (int o = 0; o < OCT; ++o) {
    const int g = il + 4 * o + rq;              // this lane's group (activation window)
    verify_a<M, KW>(sh, il + 4 * o + (col >> 2), rq, col, av);
    vf32x4 xs4[SETS];
#pragma unroll
    for (int st = 0; st < SETS; ++st) xs4[st] = *reinterpret_cast<const vf32x4*>(&sh.gs[g][st][0]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      u32x4 w = q.w[rt][o];
      if constexpr (QL) {
        w = u32x4{to_mfma_lane(w[0], src), to_mfma_lane(w[1], src), to_mfma_lane(w[2], src),
                  to_mfma_lane(w[3], src)};
      }
      const uint32_t szw = szb[rt][col][iz + 4 * o + rq];
      FmtInt4::D d;
      FmtInt4::decode(w, d, kc);
      const float s = __uint_as_float(szw << 16);
      const float zb = fmaf(-128.0f, s, __uint_as_float(szw & 0xFFFF0000u));
#pragma unroll
      for (int st = 0; st < SETS; ++st) {
        vf32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t bv[4] = {d.t[4 * j], d.t[4 * j + 1], d.t[4 * j + 2], d.t[4 * j + 3]};
          acc = mfma16x16x32(av[st][j], bv, acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (4 * st + r < M) y[rt][st][r] = fmaf(zb, xs4[st][r], fmaf(s, acc[r], y[rt][st][r]));
        }
      }
      // SB: finish one chunk before the next is decoded, which bounds the
      // registers in flight (the other waves of the CU hide the latency)
      if constexpr (SB) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Sums the four k-slots of each column (lanes col, col + 16, col + 32,
// col + 48) in a fixed order and stores the block's rows; zeroes y.
template <int M, int RT, int SETS>
__device__ __forceinline__ void verify_store(const GemvArgs& a, int64_t blk, int rq, int col,
                                             float (&y)[RT][SETS][4]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int st = 0; st < SETS; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (4 * st + r >= M) continue;
        float v = y[rt][st][r];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        y[rt][st][r] = v;
      }
    const int64_t row = (blk * RT + rt) * 16 + col;
    if (rq == 0 && row < a.n) {
#pragma unroll
      for (int st = 0; st < SETS; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * st + r;
          if (t >= M) continue;
          if (a.y32) *gmem(a.y32 + ((int64_t)t * a.n + row)) = y[rt][st][r];
          if (a.y16) *gmem(a.y16 + ((int64_t)t * a.n + row)) = f32_to_bf16(y[rt][st][r]);
        }
    }
#pragma unroll
    for (int st = 0; st < SETS; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[rt][st][r] = 0.0f;
  }
}

// mats: per-matrix descriptors (batch = one block of RT 16-row tiles;
// `chunks` = groups per row); wg_begin[g] .. wg_begin[g + 1]: workgroup g's
// global blocks, starting in matrix wg_mat[g].
template <int M, int KW, int WAVES, int RT, int OCT, bool PF, bool QL, bool SB>
__global__ __launch_bounds__(WAVES * 64) void gemm_verify_step_kernel(const GemvArgs* __restrict__ mats,
                                                                      const int64_t* __restrict__ wg_begin,
                                                                      const int32_t* __restrict__ wg_mat) {
  constexpr int SETS = VerifyShared<M, KW>::kSets;
  constexpr int GI = 4 * OCT;          // groups per item
  constexpr int IW = kSzWin / GI;      // items per (scale, zero) window
  static_assert(kSzWin % GI == 0 && KW % kSzWin == 0, "windows must nest");
  __shared__ VerifyShared<M, KW> sh;
  __shared__ __attribute__((aligned(16))) uint32_t szs[WAVES][RT][16][kSzRow];
  __shared__ int ctr;
  const int lane = lane_id();
  const int wave = wave_id();
  const int rq = lane >> 4;
  const int col = lane & 15;
  uint32_t (*szb)[16][kSzRow] = szs[wave];
  const FmtInt4::K kc = FmtInt4::consts();
  uint32_t av[SETS][4][4];
#pragma unroll
  for (int st = 0; st < SETS; ++st)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) av[st][j][e] = 0u;
  float y[RT][SETS][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int st = 0; st < SETS; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[rt][st][r] = 0.0f;
  int64_t gb = wg_begin[blockIdx.x];
  const int64_t gend = wg_begin[blockIdx.x + 1];
  int mi = wg_mat[blockIdx.x];
  while (gb < gend) {
    const GemvArgs a = mats[mi];
    const int64_t mend = a.batch_begin + a.batches;
    const int64_t lb = gb - a.batch_begin;
    const int64_t le = (gend < mend ? gend : mend) - a.batch_begin;
    const int groups = a.chunks;
    if (groups <= KW) {
      // one activation window: stage once, waves claim whole-row blocks
      const int items = (groups + GI - 1) / GI;
      __syncthreads();
      verify_stage<M, KW, WAVES * 64>(a, 0, items * GI, sh);
      if (threadIdx.x == 0) ctr = 0;
      __syncthreads();
      int64_t blk = lb + claim_batch(&ctr, lane);
      if (blk < le) {
        int64_t nxt = lb + claim_batch(&ctr, lane);
        int it = 0;
        bool more = true;
        VerifyItem<RT, OCT> A, B;
        SzWindow<RT> Z;
        sz_load<RT>(a, blk, 0, lane, Z);   // first: it is consumed first
        verify_load<RT, OCT, QL>(a, blk, 0, 0, lane, A);
        // consumes item (blk, it) from `cur` after requesting the next one
        // into `nx`; the two buffers alternate, so no loaded value is copied
        // (a copy would wait for the request just made)
        auto step = [&](const VerifyItem<RT, OCT>& cur, VerifyItem<RT, OCT>& nx) {
          if (it % IW == 0) {
            // the window of this item has arrived: publish it, request the next
            sz_put<RT>(a, it * GI, lane, Z, szb);
            const bool same = it + IW < items;
            const int64_t zb = same ? blk : nxt;
            sz_load<RT>(a, zb, same ? (it + IW) * GI : 0, lane, Z, zb < le);
          }
          int64_t b2 = blk;
          int i2 = it + 1;
          if (i2 == items) {
            b2 = nxt;
            i2 = 0;
          }
          more = b2 < le;
          verify_load<RT, OCT, QL>(a, b2, 0, i2, lane, nx, more);
          if (more && i2 == 0) nxt = lb + claim_batch(&ctr, lane);
          verify_item<M, KW, RT, OCT, QL, SB>(cur, it * GI, (it % IW) * GI, rq, col, sh, szb, kc, av, y);
          if (it + 1 == items) verify_store<M, RT, SETS>(a, blk, rq, col, y);
          blk = b2;
          it = i2;
        };
        // the prefetch left in flight is drained on the way out: otherwise
        // the (never taken) CFG edge from an exit test back to the loop head
        // carries it, and every iteration would wait for all loads
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
    } else {
      // longer rows: rounds of one block per wave, activation windows staged
      // in turn
      const int64_t rounds = (le - lb + WAVES - 1) / WAVES;
      for (int64_t rd = 0; rd < rounds; ++rd) {
        const int64_t blk = lb + rd * WAVES + wave;
        const bool mine = blk < le;
        for (int g0 = 0; g0 < groups; g0 += KW) {
          const int kw = groups - g0 < KW ? groups - g0 : KW;
          const int items = (kw + GI - 1) / GI;
          __syncthreads();
          verify_stage<M, KW, WAVES * 64>(a, g0, items * GI, sh);
          __syncthreads();
          if (!mine) continue;
          VerifyItem<RT, OCT> A, B;
          SzWindow<RT> Z;
          sz_load<RT>(a, blk, g0, lane, Z);
          verify_load<RT, OCT, QL>(a, blk, g0, 0, lane, A);
          auto step = [&](int it, const VerifyItem<RT, OCT>& cur, VerifyItem<RT, OCT>& nx) {
            if (it % IW == 0) {
              sz_put<RT>(a, g0 + it * GI, lane, Z, szb);
              sz_load<RT>(a, blk, g0 + (it + IW) * GI, lane, Z, it + IW < items);
            }
            verify_load<RT, OCT, QL>(a, blk, g0, it + 1, lane, nx, it + 1 < items);
            verify_item<M, KW, RT, OCT, QL, SB>(cur, it * GI, (it % IW) * GI, rq, col, sh, szb, kc, av, y);
          };
          for (int it = 0;; it += 2) {
            step(it, A, B);
            if (it + 1 >= items) {
              wait_vmem_all();
              break;
            }
            step(it + 1, B, A);
            if (it + 2 >= items) {
              wait_vmem_all();
              break;
            }
          }
        }
        if (mine) verify_store<M, RT, SETS>(a, blk, rq, col, y);
      }
    }
    gb = a.batch_begin + le;
    ++mi;
  }
}

}  // namespace wq
