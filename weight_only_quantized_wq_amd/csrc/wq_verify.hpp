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
//     loaded itself, and it adds s * D with the group's scale.
// With 5..8 tokens A rows 8 s + t cover all tokens over TWO group slots
// (k-slots 2 s, 2 s + 1; verify_a_wide), which halves the MFMAs.  Each
// MFMA sum starts at -128 X (X the group's activation sum of the token), so
// the decode's 128 offset cancels inside it, group by group; the lane adds
// s * (D - 128 X), and the zero points, z X summed over 32 groups, are one
// more MFMA per 32 groups (verify_zero_term).
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

#include "wq_claim.hpp"
#include "wq_formats.hpp"
#include "wq_step_shared.hpp"

namespace wq {

// Longest row (inputs) the verify kernel accepts (offsets stay in 32 bits).
constexpr int kVerifyMaxK = 131072;

// Per token count: waves per workgroup, 16-row tiles per block, quads per
// item, groups per staged activation window, code tiles in LDS (chosen by
// timing the Llama-3.1-70B verify sets; the windows of 6..8 tokens leave room
// for the tiles).
template <int M>
struct VerifyConfig {
  static constexpr int kWaves = M == 4 ? 12 : 8;
  static constexpr int kRT = 2;
  static constexpr int kOct = M == 4 ? 2 : 4;
  static constexpr int kKW = M == 2 ? 512 : (M == 6 ? 224 : (M == 7 ? 192 : (M == 8 ? 160 : 256)));
  static constexpr bool kLT = true;
};

typedef __bf16 vbf16x8 __attribute__((ext_vector_type(8)));
typedef float vf32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Activations of one K window for up to M tokens.  Token rows are padded by
// 16 bytes so the four tokens one k-slot reads sit in different banks.
template <int M, int KW>
struct alignas(16) VerifyShared {
  static constexpr int kSets = (M + 3) / 4;
  // 5..8 tokens: one MFMA serves all tokens over two group slots ("wide");
  // A operands [pair][half] instead of [set][MFMA], one accumulator set per
  // lane (its four tokens)
  static constexpr bool kWide = M > 4;
  static constexpr int kA1 = kWide ? 2 : kSets;
  static constexpr int kA2 = kWide ? 2 : 4;
  static constexpr int kYS = kWide ? 1 : kSets;
  static constexpr int kRow = KW * 16 + 4;
  static constexpr int kZLo = kWide ? 8 : 4;      // A rows of the zero-point products: part * kZLo + token
  static constexpr int kZRows = 3 * kZLo;
  static constexpr int kSumRow = KW + 8;          // bf16 per row of xz (rows 16 bytes apart in bank)
  uint32_t xs[M][kRow];          // pre-permuted bf16 pairs, 16 words per group
  float gs[KW][kSets][4];        // -128 x the per-group activation sums, [group][set][token in set]
  // the per-group activation sums X as three bf16 parts hi + mid + lo
  // (|X - hi - mid - lo| <= 2^-27 |X|), row M part + token: only the M
  // tokens' rows are kept (the A rows of absent tokens are zero registers)
  alignas(16) uint16_t xz[3 * M][kSumRow];
};

template <int RT, int OCT>
struct VerifyItem {
  u32x4 w[RT][OCT];      // codes of OCT consecutive groups of one row of each of RT tiles
};

// (scale, zero) words of the 16 rows of each tile for a window of kSzWin
// groups, loaded with 4 consecutive words per lane (a quad of lanes covers
// 64 contiguous bytes of a row) and passed through a per-wave LDS buffer,
// from which each lane reads the word of its own (row, group).  A load whose
// lanes each fetch one word of a different row would touch a cache line per
// lane; the address path, not HBM, would then set the pace.
constexpr int kSzWin = 32;
constexpr int kSzRow = kSzWin + 4;            // LDS words per row (16-byte aligned, skewed banks)
constexpr int kSzLanesPerRow = kSzWin / 4;
constexpr int kSzRowsPerLoad = kWave / kSzLanesPerRow;
constexpr int kSzLoads = 16 / kSzRowsPerLoad;
static_assert(kSzWin % 4 == 0 && 16 % kSzRowsPerLoad == 0, "window must split into whole-row loads");

template <int RT>
struct SzWindow {
  u32x4 r[RT][kSzLoads];   // load h: row kSzRowsPerLoad h + lane / kSzLanesPerRow, groups 4 (lane % ..) + 0..3
};

__device__ __forceinline__ vf32x4 mfma16x16x32(const uint32_t (&a)[4], const uint32_t (&b)[4], vf32x4 c) {
  const u32x4 av = {a[0], a[1], a[2], a[3]};
  const u32x4 bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(vbf16x8, av), __builtin_bit_cast(vbf16x8, bv), c,
                                                 0, 0, 0);
}

// The LDS entries of token t (< M) for window group g: its pre-permuted
// pairs and -128 x its sum (g < kpad), and the sum's three bf16 parts.
template <int M, int KW>
__device__ __forceinline__ void verify_put(VerifyShared<M, KW>& sh, int t, int g, int kpad, const FmtInt4::X& xv) {
  if (g < kpad) {
#pragma unroll
    for (int h = 0; h < 4; ++h)
      *reinterpret_cast<u32x4*>(&sh.xs[t][16 * g + 4 * h]) =
          u32x4{xv.p[4 * h], xv.p[4 * h + 1], xv.p[4 * h + 2], xv.p[4 * h + 3]};
    sh.gs[g][t >> 2][t & 3] = -128.0f * xv.gsum;
  }
  // each difference is exact in fp32
  const uint16_t hi = f32_to_bf16(xv.gsum);
  const float r1 = xv.gsum - __uint_as_float((uint32_t)hi << 16);
  const uint16_t mid = f32_to_bf16(r1);
  const uint16_t lo = f32_to_bf16(r1 - __uint_as_float((uint32_t)mid << 16));
  sh.xz[t][g] = hi;
  sh.xz[M + t][g] = mid;
  sh.xz[2 * M + t][g] = lo;
}

// Stages groups [g0, g0 + kpad) of every token and their sums over whole
// (scale, zero) windows (kpad rounded up to kSzWin); groups at or past the
// row's end are zero.
template <int M, int KW, int THREADS>
__device__ __forceinline__ void verify_stage(const GemvArgs& a, int g0, int kpad, VerifyShared<M, KW>& sh) {
  constexpr int SETS = VerifyShared<M, KW>::kSets;
  constexpr int ZLO = VerifyShared<M, KW>::kZLo;
  const int kz = (kpad + kSzWin - 1) / kSzWin * kSzWin;
#pragma unroll 1
  for (int it = threadIdx.x; it < ZLO * kz; it += THREADS) {
    const int t = it / kz;
    const int g = it - t * kz;
    const int gg = g0 + g;
    if (t < M) {
      verify_put<M, KW>(sh, t, g, kpad, FmtInt4::load_x(a.x + (int64_t)t * a.k, gg, gg < a.chunks && g < kpad));
    } else if (t < 4 * SETS && g < kpad) {
      sh.gs[g][t >> 2][t & 3] = 0.0f;
    }
  }
}

// Two-phase staging of one whole window [0, kz) (kz a multiple of kSzWin):
// stage_issue requests this thread's pieces (token, group) of the M token
// rows -- through a buffer resource over them, so pieces past a row read as
// zero without a branch -- and stage_finish permutes them into LDS.  Issued
// before the weights, the activations arrive first, and their wait does not
// hold for the weight loads behind them.
template <int M, int KW, int THREADS>
struct VerifyStage2 {
  static constexpr int kPieces = (M * KW + THREADS - 1) / THREADS;
  u32x4 v[kPieces][4];

  __device__ __forceinline__ void issue(const GemvArgs& a, int kz) {
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(a.x, (uint32_t)(M * a.k * 2));
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
      const int it = (int)threadIdx.x + q * THREADS;
      const int t = it / kz, g = it - (it / kz) * kz;
      const bool ok = t < M && g < a.chunks;
      const uint32_t off = ok ? (uint32_t)t * (uint32_t)(a.k * 2) + (uint32_t)g * 64u : 0x80000000u;
#pragma unroll
      for (int h = 0; h < 4; ++h) v[q][h] = buffer_load16(rx, off + 16u * h);
    }
  }
  __device__ __forceinline__ void finish(VerifyShared<M, KW>& sh, int kz) const {
    constexpr int SETS = VerifyShared<M, KW>::kSets;
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
      const int it = (int)threadIdx.x + q * THREADS;
      const int t = it / kz, g = it - (it / kz) * kz;
      if (t < M) verify_put<M, KW>(sh, t, g, kz, FmtInt4::from_words(v[q]));
    }
    // tokens past M in the last set: zero sums
    for (int it = threadIdx.x; it < (4 * SETS - M) * kz; it += THREADS) {
      const int t = M + it / kz, g = it - (it / kz) * kz;
      sh.gs[g][t >> 2][t & 3] = 0.0f;
    }
  }
};

// The zero points of a (scale, zero) window for the wave's block.  A group
// contributes s * (D - 128 X) + z * X to each token (D = sum of (128 + q) x
// from the MFMAs, whose accumulators start at -128 X, X the group's
// activation sum); the z * X terms of the window's 32 groups are MFMAs with
// A = X (rows kZLo part + t: its hi, mid and lo bf16 parts), B = the groups'
// zero points (bf16, exact), one MFMA per 16 A rows.  Lane (rq, col)
// receives rows 4 rq + r of each: in the wide layout tokens 4 (rq % 2) + r
// (hi or mid in the first MFMA, lo or nothing in the second); with up to four
// tokens token r (hi, mid, lo or nothing by rq) -- in both the tokens of its
// own accumulators, so the slot sums of the fold add the parts.  il: the
// window's first group in the activation window; chunk i of the window uses
// (scale, zero) word i >> gshift.
template <int M, int KW, int RT, int YS>
__device__ __forceinline__ void verify_zero_term(const VerifyShared<M, KW>& sh, const uint32_t (*szb)[16][kSzRow],
                                                 int il, int gshift, int rq, int col, float (&y)[RT][YS][4]) {
  static_assert(YS == 1, "one accumulator set per lane (at most four tokens, or the wide layout)");
  // the window's words were stored by other lanes of the wave (sz_put)
  __builtin_amdgcn_wave_barrier();
  constexpr int ZR = VerifyShared<M, KW>::kZRows;
  constexpr int ZM = (ZR + 15) / 16;   // MFMAs per tile
  uint32_t av[ZM][4];
  constexpr int ZLO = VerifyShared<M, KW>::kZLo;
#pragma unroll
  for (int h = 0; h < ZM; ++h) {
    const int row = 16 * h + col;      // A row ZLO part + token
    const int part = row / ZLO, t = row % ZLO;
    av[h][0] = av[h][1] = av[h][2] = av[h][3] = 0u;
    if (row < ZR && t < M) {
      const u32x4 xa = *reinterpret_cast<const u32x4*>(&sh.xz[row < ZR && t < M ? M * part + t : 0][il + 8 * rq]);
      av[h][0] = xa[0];
      av[h][1] = xa[1];
      av[h][2] = xa[2];
      av[h][3] = xa[3];
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    uint32_t w[8];
    if (gshift == 0) {
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(&szb[rt][col][8 * rq]);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(&szb[rt][col][8 * rq + 4]);
      w[0] = w0[0]; w[1] = w0[1]; w[2] = w0[2]; w[3] = w0[3];
      w[4] = w1[0]; w[5] = w1[1]; w[6] = w1[2]; w[7] = w1[3];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = szb[rt][col][(8 * rq + i) >> gshift];
    }
    uint32_t bz[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bz[j] = __builtin_amdgcn_perm(w[2 * j + 1], w[2 * j], 0x07060302u);   // (z_2j, z_2j+1)
    vf32x4 dz = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int h = 0; h < ZM; ++h) dz = mfma16x16x32(av[h], bz, dz);
#pragma unroll
    for (int r = 0; r < 4; ++r) y[rt][0][r] += dz[r];
  }
}

// Loads the codes of item `it` of window [g0, ...) of block `blk` (tiles
// RT blk .. RT blk + RT - 1): OCT quads of 4 consecutive groups (k-slot s of
// quad o = group 4 o + s of the item) for the 16 rows of each tile, in one of
// two layouts:
//   * LT (line-wide; OCT even): load o reads rows 8 (o % 2) + lane / 8,
//     group 8 (o / 2) + lane % 8 -- 128 contiguous bytes of each of 8 rows,
//     the shape that streams at full rate -- and verify_item moves the codes
//     to their MFMA lanes through a per-wave LDS tile;
//   * otherwise each quad of lanes reads ONE row (lane (row = lane / 4,
//     k-slot = lane % 4)), 64 bytes of each of 16 rows per load, and
//     verify_item moves each word to the MFMA lane (k-slot = lane / 16, row =
//     lane % 16) with a cross-lane permute.
// Rows past n and groups past the row read as zero, and so does everything
// with !any: the loads are issued on every path, so code after a conditional
// prefetch waits only for the item it consumes.
template <int RT, int OCT, bool LT>
__device__ __forceinline__ void verify_load(const GemvArgs& a, int64_t blk, int g0, int it, int lane,
                                            VerifyItem<RT, OCT>& q, bool any = true) {
  static_assert(!LT || OCT % 2 == 0, "line-wide loads come in pairs");
  const uint32_t row_bytes = (uint32_t)a.row_bytes;
  const int g_item = g0 + it * 4 * OCT;
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
      const int lrow = LT ? 8 * (o & 1) + (lane >> 3) : lane >> 2;
      const int g = LT ? g_item + 8 * (o >> 1) + (lane & 7) : g_item + 4 * o + (lane & 3);
      const bool ok = g < a.chunks;
      q.w[rt][o] = buffer_load16_nt(rw, ok ? (uint32_t)lrow * row_bytes + (uint32_t)g * 16u : 0x80000000u);
    }
  }
}

// Loads the (scale, zero) words of chunks [gw, gw + kSzWin) of block `blk`
// (zeros with !any).  With groups of G = 32 << gshift inputs (gshift =
// kPerRowShift: one group per row) chunk c uses word c >> gshift of its row;
// gw is a multiple of kSzWin, so the window's words start at word
// gw >> gshift and chunk gw + i uses word i >> gshift of the window (the
// window then holds more words than its chunks use).
// OPAQUE hides each offset's select from the compiler, which otherwise may
// issue two loads into the same registers under complementary lane masks;
// the second then waits for every load in flight.
template <int RT, bool OPAQUE = false>
__device__ __forceinline__ void sz_load(const GemvArgs& a, int64_t blk, int gw, int lane, SzWindow<RT>& z,
                                        bool any = true) {
  const uint32_t words = (uint32_t)int4_row_words(a.chunks, a.gshift);
  const int g = (gw >> a.gshift) + 4 * (lane % kSzLanesPerRow);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t rbase = (blk * RT + rt) * 16;
    const int64_t left = a.n - rbase;
    const bool live = any && left > 0;
    const uint32_t rows_ok = !live ? 0u : (left >= 16 ? 16u : (uint32_t)left);
    const int64_t rb = live ? rbase : 0;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.sz + rb * words, rows_ok * words * 4u);
#pragma unroll
    for (int h = 0; h < kSzLoads; ++h) {
      const uint32_t row = (uint32_t)(kSzRowsPerLoad * h + lane / kSzLanesPerRow);
      int off = (uint32_t)g < words ? (int)((row * words + (uint32_t)g) * 4u) : (int)0x80000000;
      if constexpr (OPAQUE) asm volatile("" : "+v"(off));
      z.r[rt][h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2));
    }
  }
}

// Writes a loaded window into the wave's LDS buffer; words past the row's
// last (which belong to the next row) become zero.
template <int RT>
__device__ __forceinline__ void sz_put(const GemvArgs& a, int gw, int lane, const SzWindow<RT>& z,
                                       uint32_t (*buf)[16][kSzRow]) {
  const int64_t words = int4_row_words(a.chunks, a.gshift);
  const int g = (gw >> a.gshift) + 4 * (lane % kSzLanesPerRow);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int h = 0; h < kSzLoads; ++h) {
      u32x4 v = z.r[rt][h];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (g + e >= words) v[e] = 0u;
      *reinterpret_cast<u32x4*>(&buf[rt][kSzRowsPerLoad * h + lane / kSzLanesPerRow][4 * (lane % kSzLanesPerRow)]) = v;
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
                                         uint32_t (&av)[VerifyShared<M, KW>::kA1][VerifyShared<M, KW>::kA2][4]) {
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

// Wide layout (5..8 tokens): A row 8 s + t is token t restricted to group
// slot s (k-slots 2 s and 2 s + 1).  MFMA (pair p, half h) of quad [gq, gq +
// 4) covers groups gq + 2 p + s, k-slot 2 s + e holding 32-bit code word
// 2 e + h of its group -- inputs 8 (2 e + h) .. + 7, activation pair words
// 4 (2 e + h) .. + 3.  Lane (rq, col) carries data when col / 8 == rq / 2
// (its slot) and token col % 8 exists; the others keep zeros and read nothing.
template <int M, int KW>
__device__ __forceinline__ void verify_a_wide(const VerifyShared<M, KW>& sh, int gq, int rq, int col,
                                              uint32_t (&av)[2][2][4]) {
  const int s = rq >> 1, e = rq & 1, t = col & 7;
  if ((col >> 3) == s && t < M) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int ga = gq + 2 * p + s;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(&sh.xs[t < M ? t : 0][16 * ga + 8 * e + 4 * h]);
        av[p][h][0] = v[0];
        av[p][h][1] = v[1];
        av[p][h][2] = v[2];
        av[p][h][3] = v[3];
      }
    }
  }
}

// LT: a 16-row x 128-byte tile of codes per wave.  The 16-byte slots of a
// row are XOR-swizzled by row pair (slot p of row r at p ^ (r / 2 % 8)), so
// the stores (two rows of 8 slots per 16 lanes) and the reads (one slot of
// 16 rows) fall in distinct banks.
constexpr int kVerifyTile = 16 * 128;
__device__ __forceinline__ int verify_tile_at(int row, int slot) { return row * 128 + ((slot ^ ((row >> 1) & 7)) << 4); }

// Wide layout (5..8 tokens; see verify_a_wide): before quads o and o + 1
// (o even) each tile's loads o and o + 1 pass through the wave's LDS tile as
// in the four-token layout, and lane (rq, col) reads back, for quad o + h and
// pair p, bytes 8 e .. 8 e + 7 (code words 2 e and 2 e + 1) of group
// 4 h + 2 p + rq / 2 of row col (e = rq % 2).  D rows 8 s + 4 e + r of column
// col: tokens 4 e + r of (row col, group 2 p + s) minus 128 X, scaled by the
// lane's own scale (z X comes from verify_zero_term).  Tokens past M have
// zero activations and sums, so their accumulators stay zero and are never
// stored.
template <int M, int KW, int RT, int OCT>
__device__ __forceinline__ void verify_item_wide(const VerifyItem<RT, OCT>& q, int il, int iz, int gshift, int rq,
                                                 int col, const VerifyShared<M, KW>& sh,
                                                 const uint32_t (*szb)[16][kSzRow], const FmtInt4::K& kc,
                                                 uint32_t (&av)[2][2][4], float (&y)[RT][1][4], uint8_t* tile) {
  static_assert(OCT % 2 == 0, "line-wide loads come in pairs");
  const int wr = rq * 2 + (col >> 3), ws = col & 7;   // tile store: row wr (+ 8), slot ws (lane = 16 rq + col)
  const int s = rq >> 1, e = rq & 1;
  u32x2 wl[RT][2][2];
#pragma unroll
  for (int o = 0; o < OCT; ++o) {
    if ((o & 1) == 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        // lanes read what other lanes stored: the wave barriers keep the
        // compiler from reordering these LDS accesses across lanes' roles
        __builtin_amdgcn_wave_barrier();
        *reinterpret_cast<u32x4*>(tile + verify_tile_at(wr, ws)) = q.w[rt][o];
        *reinterpret_cast<u32x4*>(tile + verify_tile_at(wr + 8, ws)) = q.w[rt][o + 1];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int p = 0; p < 2; ++p)
            wl[rt][h][p] = *reinterpret_cast<const u32x2*>(tile + verify_tile_at(col, 4 * h + 2 * p + s) + 8 * e);
      }
    }
    verify_a_wide<M, KW>(sh, il + 4 * o, rq, col, av);
    vf32x4 c0[2];   // -128 X of the lane's tokens and group: the MFMA sums start there
#pragma unroll
    for (int p = 0; p < 2; ++p) c0[p] = *reinterpret_cast<const vf32x4*>(&sh.gs[il + 4 * o + 2 * p + s][e][0]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const float sc = __uint_as_float(szb[rt][col][(iz + 4 * o + 2 * p + s) >> gshift] << 16);
        vf32x4 acc = c0[p];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t v = wl[rt][o & 1][p][h];
          const uint32_t bv[4] = {(v & kc.mask) | FmtInt4::kMagic, ((v >> 4) & kc.mask) | FmtInt4::kMagic,
                                  ((v >> 8) & kc.mask) | FmtInt4::kMagic, ((v >> 12) & kc.mask) | FmtInt4::kMagic};
          acc = mfma16x16x32(av[p][h], bv, acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) y[rt][0][r] = fmaf(sc, acc[r], y[rt][0][r]);
      }
    }
  }
}

// Accumulates one item into y[tile][set][token]; `il` is the item's first
// chunk within the staged activation window and `iz` within the (scale,
// zero) window held in `szb`, where chunk iz + i takes word (iz + i) >> gshift.
// LT: before quads o and o + 1 (o even), each tile's loads o and o + 1 (16
// rows x 8 groups) pass through the wave's LDS `tile`, and each lane reads
// back its (row col, group 4 (o % 2) + rq) chunks of the two quads; the
// wave's LDS accesses complete in order, so the next tile's stores never
// overtake these reads.
template <int M, int KW, int RT, int OCT, bool LT>
__device__ __forceinline__ void verify_item(const VerifyItem<RT, OCT>& q, int il, int iz, int gshift, int rq,
                                            int col, const VerifyShared<M, KW>& sh, const uint32_t (*szb)[16][kSzRow],
                                            const FmtInt4::K& kc,
                                            uint32_t (&av)[VerifyShared<M, KW>::kA1][VerifyShared<M, KW>::kA2][4],
                                            float (&y)[RT][VerifyShared<M, KW>::kYS][4], uint8_t* tile) {
  constexpr int SETS = VerifyShared<M, KW>::kSets;
  if (iz == 0) verify_zero_term<M, KW, RT, VerifyShared<M, KW>::kYS>(sh, szb, il, gshift, rq, col, y);
  if constexpr (VerifyShared<M, KW>::kWide) {
    static_assert(LT, "the wide layout reads its codes from the LDS tile");
    verify_item_wide<M, KW, RT, OCT>(q, il, iz, gshift, rq, col, sh, szb, kc, av, y, tile);
    return;
  } else {
  const int src = (4 * col + rq) * 4;   // byte address of the lane holding this lane's codes (!LT)
  const int wr = rq * 2 + (col >> 3), ws = col & 7;   // LT store: row wr (+ 8), slot ws (lane = 16 rq + col)
  u32x4 wl[RT][2];
#pragma unroll
  for (int o = 0; o < OCT; ++o) {
    if constexpr (LT) {
      if ((o & 1) == 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          // lanes read what other lanes stored: the wave barriers keep the
          // compiler from reordering these LDS accesses across lanes' roles
          __builtin_amdgcn_wave_barrier();
          *reinterpret_cast<u32x4*>(tile + verify_tile_at(wr, ws)) = q.w[rt][o];
          *reinterpret_cast<u32x4*>(tile + verify_tile_at(wr + 8, ws)) = q.w[rt][o + 1];
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int h = 0; h < 2; ++h) wl[rt][h] = *reinterpret_cast<const u32x4*>(tile + verify_tile_at(col, 4 * h + rq));
        }
      }
    }
    verify_a<M, KW>(sh, il + 4 * o + (col >> 2), rq, col, av);
    vf32x4 c0[SETS];   // -128 X of the lane's tokens and group: the MFMA sums start there
#pragma unroll
    for (int st = 0; st < SETS; ++st) c0[st] = *reinterpret_cast<const vf32x4*>(&sh.gs[il + 4 * o + rq][st][0]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      u32x4 w = q.w[rt][o];
      if constexpr (LT) {
        w = wl[rt][o & 1];
      } else {
        w = u32x4{to_mfma_lane(w[0], src), to_mfma_lane(w[1], src), to_mfma_lane(w[2], src),
                  to_mfma_lane(w[3], src)};
      }
      const uint32_t szw = szb[rt][col][(iz + 4 * o + rq) >> gshift];
      FmtInt4::D d;
      FmtInt4::decode(w, d, kc);
      const float s = __uint_as_float(szw << 16);
#pragma unroll
      for (int st = 0; st < SETS; ++st) {
        vf32x4 acc = c0[st];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t bv[4] = {d.t[4 * j], d.t[4 * j + 1], d.t[4 * j + 2], d.t[4 * j + 3]};
          acc = mfma16x16x32(av[st][j], bv, acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (4 * st + r < M) y[rt][st][r] = fmaf(s, acc[r], y[rt][st][r]);
        }
      }
    }
  }
  }
}

// Rounds of blocks for rows longer than one activation window: each window
// is staged once per round and the round's blocks are claimed for it; the
// sums of a block's finished windows wait in LDS (VerifyPart).
template <int WAVES>
constexpr int verify_round_blocks() { return WAVES; }

template <int M, int RT, int SR>
struct VerifyPart {
  float v[SR][RT * 16][M];
};

// Block `blk` (index `bi` of its round) has streamed the window: sums the
// four k-slots of each column (lanes col, col + 16, col + 32, col + 48) in a
// fixed order, adds the block's earlier windows (!first) and stores the rows
// (last) or keeps the running sum for the next window; zeroes y.  The sum of
// a row is taken window by window in order, whichever wave streams them.
// Wide layout: lanes col + 16 e and col + 16 (2 + e) hold the two group
// slots of tokens 4 e + r.
template <int M, int RT, int SETS, int SR>
__device__ __forceinline__ void verify_fold(const GemvArgs& a, int64_t blk, int bi, bool first, bool last, int rq,
                                            int col, float (&y)[RT][SETS][4], VerifyPart<M, RT, SR>& part) {
  if constexpr (M > 4) {
    static_assert(SETS == 1, "wide accumulators: one set of four tokens per lane");
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) y[rt][0][r] += __shfl_xor(y[rt][0][r], 32);
      const int64_t row = (blk * RT + rt) * 16 + col;
      if (rq < 2) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * rq + r;
          if (t >= M) continue;
          float v = y[rt][0][r];
          if (!first) v = part.v[bi][rt * 16 + col][t] + v;
          if (!last) {
            part.v[bi][rt * 16 + col][t] = v;
          } else if (row < a.n) {
            if (a.y32) *gmem(a.y32 + ((int64_t)t * a.n + row)) = v;
            if (a.y16) *gmem(a.y16 + ((int64_t)t * a.n + row)) = f32_to_bf16(v);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) y[rt][0][r] = 0.0f;
    }
    return;
  }
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
    if (rq == 0) {
#pragma unroll
      for (int st = 0; st < SETS; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * st + r;
          if (t >= M) continue;
          float v = y[rt][st][r];
          if (!first) v = part.v[bi][rt * 16 + col][t] + v;
          if (!last) {
            part.v[bi][rt * 16 + col][t] = v;
          } else if (row < a.n) {
            if (a.y32) *gmem(a.y32 + ((int64_t)t * a.n + row)) = v;
            if (a.y16) *gmem(a.y16 + ((int64_t)t * a.n + row)) = f32_to_bf16(v);
          }
        }
    }
#pragma unroll
    for (int st = 0; st < SETS; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[rt][st][r] = 0.0f;
  }
}

// The waves' share of one activation window: blocks [b0, b1) of matrix `a`,
// claimed one at a time from `ctr` (zeroed by the caller); each streams the
// window's `items` items (groups [g0, g0 + GI items)) and folds its sums
// (verify_fold).  The next item's loads are issued before the current one is
// reduced, across block boundaries too; the two item buffers alternate, so
// no loaded value is copied (a copy would wait for the loads just issued).
template <int M, int KW, int WAVES, int RT, int OCT, int SR, bool LT>
__device__ __forceinline__ void verify_window(const GemvArgs& a, int64_t b0, int64_t b1, int g0, int items,
                                              bool first, bool last, int* ctr, int lane, int rq, int col,
                                              const VerifyShared<M, KW>& sh, uint32_t (*szb)[16][kSzRow],
                                              const FmtInt4::K& kc,
                                              uint32_t (&av)[VerifyShared<M, KW>::kA1][VerifyShared<M, KW>::kA2][4],
                                              float (&y)[RT][VerifyShared<M, KW>::kYS][4],
                                              VerifyPart<M, RT, SR>& part, uint8_t* tile) {
  constexpr int YS = VerifyShared<M, KW>::kYS;
  constexpr int GI = 4 * OCT;          // groups per item
  constexpr int IW = kSzWin / GI;      // items per (scale, zero) window
  const int64_t nb = b1 - b0;
  int64_t bi = claim_batch(ctr, lane);
  if (bi >= nb) return;
  int64_t nxt = claim_batch(ctr, lane);
  int it = 0;
  bool more = true;
  VerifyItem<RT, OCT> A, B;
  SzWindow<RT> Z;
  sz_load<RT>(a, b0 + bi, g0, lane, Z);   // first: it is consumed first
  verify_load<RT, OCT, LT>(a, b0 + bi, g0, 0, lane, A);
  // consumes item (bi, it) from `cur` after requesting the next one into `nx`
  auto step = [&](const VerifyItem<RT, OCT>& cur, VerifyItem<RT, OCT>& nx) {
    if (it % IW == 0) {
      // the window of this item has arrived: publish it, request the next
      sz_put<RT>(a, g0 + it * GI, lane, Z, szb);
      const bool same = it + IW < items;
      const int64_t zb = same ? bi : nxt;
      sz_load<RT>(a, b0 + zb, g0 + (same ? (it + IW) * GI : 0), lane, Z, zb < nb);
    }
    int64_t b2 = bi;
    int i2 = it + 1;
    if (i2 == items) {
      b2 = nxt;
      i2 = 0;
    }
    more = b2 < nb;
    verify_load<RT, OCT, LT>(a, b0 + b2, g0, i2, lane, nx, more);
    if (more && i2 == 0) nxt = claim_batch(ctr, lane);
    verify_item<M, KW, RT, OCT, LT>(cur, it * GI, (it % IW) * GI, a.gshift, rq, col, sh, szb, kc, av, y, tile);
    if (it + 1 == items) verify_fold<M, RT, YS, SR>(a, b0 + bi, (int)bi, first, last, rq, col, y, part);
    bi = b2;
    it = i2;
  };
  // the prefetch left in flight is drained on the way out: otherwise the
  // (never taken) CFG edge from an exit test back to the loop head carries
  // it, and every iteration would wait for all loads
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

// Balance between rows within one activation window ("short") and longer
// rows ("long"), which stream more slowly per byte (window rounds with a
// barrier each, rows further apart).  Ranges are cut in cost units in which
// a long-row byte costs f short-row bytes.  Each launch measures the time its
// workgroups spend on each kind and the last one to finish moves f a quarter
// of the way to the measured ratio of the two rates (clamped to [0.5, 4]);
// the next launch cuts with it.  Which workgroup computes a row never changes
// the row's result.
//
// On top of that, ranges follow the measured speeds of the workgroups, as in
// the one-token step (StepBalance, step_balance_update).
struct VerifyBalance {
  double f;
  double t[2];      // this launch: wall-clock ticks spent on short / long rows
  double c[2];      // this launch: bytes of short / long rows streamed
  double pad;
};

struct VerifyCuts {
  const double* pre_short;   // [count + 1] bytes of short-row matrices before matrix i
  const double* pre_long;    // [count + 1] bytes of long-row matrices before matrix i
  const double* bcost;       // [count] bytes of one block of matrix i
  VerifyBalance* bal;
  StepBalance* wg;           // per-workgroup speeds and shares
  int32_t count;
};

// mats: per-matrix descriptors (batch = one block of RT 16-row tiles;
// `chunks` = groups per row).  Each workgroup cuts its own contiguous range
// of the step's blocks from the cost prefixes and the balance factor.
template <int M, int KW, int WAVES, int RT, int OCT, bool LT>
__global__ __launch_bounds__(WAVES * 64) void gemm_verify_step_kernel(const GemvArgs* __restrict__ mats,
                                                                      VerifyCuts cuts) {
  constexpr int GI = 4 * OCT;          // groups per item
  constexpr int SR = verify_round_blocks<WAVES>();
  static_assert(kSzWin % GI == 0 && KW % kSzWin == 0, "windows must nest");
  __shared__ VerifyShared<M, KW> sh;
  __shared__ __attribute__((aligned(16))) uint32_t szs[WAVES][RT][16][kSzRow];
  __shared__ VerifyPart<M, RT, SR> part;
  __shared__ __attribute__((aligned(16))) uint8_t tiles[LT ? WAVES : 1][LT ? kVerifyTile : 16];
  __shared__ int ctr;
  __shared__ int64_t range[2];
  __shared__ int first_mat;
  const int lane = lane_id();
  const int wave = wave_id();
  const int rq = lane >> 4;
  const int col = lane & 15;
  uint32_t (*szb)[16][kSzRow] = szs[wave];
  const FmtInt4::K kc = FmtInt4::consts();

  // this workgroup's range: its speed-weighted share of the step's cost
  const long long t_start = wall_clock64();
  const double f = cuts.bal->f;
  const int epoch = step_epoch(cuts.wg);
  double c0, c1;
  step_share(cuts.wg, epoch, cuts.pre_short[cuts.count] + f * cuts.pre_long[cuts.count], c0, c1);
  if (threadIdx.x == 0) {
    range[0] = mats[cuts.count - 1].batch_begin + mats[cuts.count - 1].batches;
    range[1] = range[0];
    first_mat = cuts.count - 1;
  }
  __syncthreads();
  // the block at cost c: first block of matrix i (p0 <= c < p1) whose start
  // is at or past c; every matrix is checked by one thread
  for (int i = threadIdx.x; i < cuts.count; i += WAVES * kWave) {
    const double p0 = cuts.pre_short[i] + f * cuts.pre_long[i];
    const double p1 = cuts.pre_short[i + 1] + f * cuts.pre_long[i + 1];
    const GemvArgs& m = mats[i];
    const double bc = cuts.bcost[i] * (m.chunks > KW ? f : 1.0);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const double c = e == 0 ? c0 : c1;
      if (p0 <= c && c < p1) {
        int64_t local = (int64_t)((c - p0) / bc + 0.999999);
        if (local > m.batches) local = m.batches;
        range[e] = m.batch_begin + local;
        if (e == 0) first_mat = i;
      }
    }
  }
  __syncthreads();

  constexpr int A1 = VerifyShared<M, KW>::kA1, A2 = VerifyShared<M, KW>::kA2, YS = VerifyShared<M, KW>::kYS;
  uint32_t av[A1][A2][4];
#pragma unroll
  for (int st = 0; st < A1; ++st)
#pragma unroll
    for (int j = 0; j < A2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) av[st][j][e] = 0u;
  float y[RT][YS][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int st = 0; st < YS; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[rt][st][r] = 0.0f;
  int64_t gb = uniform_i64(range[0]);
  const int64_t gend = uniform_i64(range[1]);
  int mi = __builtin_amdgcn_readfirstlane(first_mat);
  double tk[2] = {0.0, 0.0}, ck[2] = {0.0, 0.0};
  long long tprev = 0;
  int kprev = -1;
  while (gb < gend) {
    const GemvArgs a = mats[mi];
    const int64_t mend = a.batch_begin + a.batches;
    if (gb >= mend) {   // the range starts at the next matrix
      ++mi;
      continue;
    }
    const int64_t lb = gb - a.batch_begin;
    const int64_t le = (gend < mend ? gend : mend) - a.batch_begin;
    const int groups = a.chunks;
    const int kind = groups > KW;
    // time of a segment: from the barrier that opens it to the one that
    // opens the next
    __syncthreads();
    const long long now = wall_clock64();
    if (kprev >= 0) tk[kprev] += (double)(now - tprev);
    tprev = now;
    kprev = kind;
    ck[kind] += (double)(le - lb) * cuts.bcost[mi];
    // rows within one window: a single round over the whole range; longer
    // rows: rounds of SR blocks, windows staged in turn
    const int64_t span = kind ? (int64_t)SR : le - lb;
    for (int64_t r0 = lb; r0 < le; r0 += span) {
      const int64_t r1 = le - r0 < span ? le : r0 + span;
      for (int g0 = 0; g0 < groups; g0 += KW) {
        const int kw = groups - g0 < KW ? groups - g0 : KW;
        const int items = (kw + GI - 1) / GI;
        __syncthreads();
        verify_stage<M, KW, WAVES * 64>(a, g0, items * GI, sh);
        if (threadIdx.x == 0) ctr = 0;
        __syncthreads();
        verify_window<M, KW, WAVES, RT, OCT, SR, LT>(a, r0, r1, g0, items, g0 == 0, g0 + KW >= groups, &ctr,
                                                         lane, rq, col, sh, szb, kc, av, y, part,
                                                         tiles[LT ? wave : 0]);
      }
    }
    gb = a.batch_begin + le;
    ++mi;
  }
  __syncthreads();
  VerifyBalance* b = cuts.bal;
  if (threadIdx.x == 0) {
    if (kprev >= 0) tk[kprev] += (double)(wall_clock64() - tprev);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      atomicAdd(&b->t[e], tk[e]);
      atomicAdd(&b->c[e], ck[e]);
    }
  }
  // the sums above are performed before this workgroup's count (the report's
  // wait), so the last workgroup reads all of them
  static_assert(sizeof(part) >= WAVES * sizeof(double), "the partial sums' LDS holds the update's sums");
  step_balance_report<WAVES>(cuts.wg, epoch, c1 - c0, t_start, reinterpret_cast<double*>(&part), [&] {
    // the long-row factor for the next launch
    double t[2], c[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      t[e] = __hip_atomic_load(&b->t[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      c[e] = __hip_atomic_load(&b->c[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (t[0] > 0.0 && t[1] > 0.0 && c[0] > 0.0 && c[1] > 0.0) {
      double nf = 0.75 * f + 0.25 * ((t[1] / c[1]) / (t[0] / c[0]));
      nf = fmin(fmax(nf, 0.5), 4.0);
      __hip_atomic_store(&b->f, nf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      __hip_atomic_store(&b->t[e], 0.0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&b->c[e], 0.0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  });
}

// One matrix per launch (the single-matrix verify product), rows within one
// activation window (k <= 32 KW), in the claiming frame of wq_claim.hpp: a
// block is RT 16-row tiles, a unit one (scale, zero) window of kSzWin groups
// (IW items).  The activations are staged once, their loads issued before
// the first unit's weights (a wait for a load also waits for everything
// issued before it).  The next unit is claimed, and its words and first item
// requested, before the current one is reduced.
template <int M, int KW, int WAVES, int RT, int OCT, bool LT>
__global__ __launch_bounds__(WAVES * 64) void gemm_verify_matrix_kernel(GemvArgs a, MatrixClaim* claim,
                                                                        int32_t cap) {
  constexpr int GI = 4 * OCT;          // groups per item
  constexpr int IW = kSzWin / GI;      // items per unit
  constexpr int UMAX = KW / kSzWin;    // units per block at most
  constexpr int R = 2;                 // blocks whose unit sums may wait in LDS at once
  static_assert(kSzWin % GI == 0 && KW % kSzWin == 0 && IW % 2 == 0, "windows must nest, items come in pairs");
  constexpr int A1 = VerifyShared<M, KW>::kA1, A2 = VerifyShared<M, KW>::kA2, YS = VerifyShared<M, KW>::kYS;
  __shared__ VerifyShared<M, KW> sh;
  __shared__ __attribute__((aligned(16))) uint32_t szs[WAVES][RT][16][kSzRow];
  __shared__ VerifyPart<M, RT, R * UMAX> part;
  __shared__ __attribute__((aligned(16))) uint8_t tiles[LT ? WAVES : 1][LT ? kVerifyTile : 16];
  __shared__ MatrixUnitLds<R> ul;
  const int lane = lane_id();
  const int wave = wave_id();
  const int rq = lane >> 4;
  const int col = lane & 15;
  uint32_t (*szb)[16][kSzRow] = szs[wave];
  uint8_t* tile = tiles[LT ? wave : 0];
  const FmtInt4::K kc = FmtInt4::consts();
  const int ups = (a.chunks + kSzWin - 1) / kSzWin;    // units per block (1..UMAX)
  const int first = ups < WAVES ? ups : WAVES;          // units taken without a claim
  MatrixUnits<R> mu{ul, claim, ups, cap, (int)a.batches, lane};
  mu.init(wave, first);

  uint32_t av[A1][A2][4];
#pragma unroll
  for (int st = 0; st < A1; ++st)
#pragma unroll
    for (int j = 0; j < A2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) av[st][j][e] = 0u;
  float y[RT][YS][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int st = 0; st < YS; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[rt][st][r] = 0.0f;

  // the current unit (block jl of this workgroup = global block gb, window u)
  int jl = 0, u = wave, gb = (int)blockIdx.x;
  bool have = wave < first;
  VerifyItem<RT, OCT> A, B;
  SzWindow<RT> Z;
  VerifyStage2<M, KW, WAVES * 64> stage;
  stage.issue(a, ups * kSzWin);
  __builtin_amdgcn_sched_barrier(0);
  sz_load<RT, true>(a, have ? gb : 0, kSzWin * u, lane, Z, have);
  // the words before the codes, as in the loop: a window's words are then
  // older than the item in flight when they are published, on every path
  // into the loop (otherwise the wait there drains the prefetch)
  __builtin_amdgcn_sched_barrier(0);
  verify_load<RT, OCT, LT>(a, have ? gb : 0, 0, IW * u, lane, A, have);
  stage.finish(sh, ups * kSzWin);
  __syncthreads();
  if (!have) {
    have = mu.claim_next(jl, u, gb);
    sz_load<RT, true>(a, have ? gb : 0, kSzWin * u, lane, Z, have);
    __builtin_amdgcn_sched_barrier(0);
    verify_load<RT, OCT, LT>(a, have ? gb : 0, 0, IW * u, lane, A, have);
  }

  while (have) {
    int jn, un, gn;
    const bool more = mu.claim_next(jn, un, gn);
    // the current window's words have arrived: publish them, request the next
    sz_put<RT>(a, kSzWin * u, lane, Z, szb);
    sz_load<RT, true>(a, more ? gn : 0, kSzWin * un, lane, Z, more);
#pragma unroll
    for (int h = 0; h < IW; h += 2) {
      // the items' places in the window, opaque to the compiler: as
      // constants they let it hoist every word address of the window out of
      // the loop, which spills
      int iz0 = h * GI, iz1 = (h + 1) * GI;
      asm volatile("" : "+s"(iz0), "+s"(iz1));
      verify_load<RT, OCT, LT>(a, gb, 0, IW * u + h + 1, lane, B);
      verify_item<M, KW, RT, OCT, LT>(A, IW * u * GI + iz0, iz0, a.gshift, rq, col, sh, szb, kc, av, y, tile);
      if (h + 2 < IW) {
        verify_load<RT, OCT, LT>(a, gb, 0, IW * u + h + 2, lane, A);
      } else {
        verify_load<RT, OCT, LT>(a, more ? gn : 0, 0, IW * un, lane, A, more);
      }
      verify_item<M, KW, RT, OCT, LT>(B, IW * u * GI + iz1, iz1, a.gshift, rq, col, sh, szb, kc, av, y, tile);
    }
    // this unit's sums into its slot, once the slot's previous block is out
    const int sl = jl % R;
    mu.wait_slot(jl);
    verify_fold<M, RT, YS, R * UMAX>(a, gb, sl * UMAX + u, true, false, rq, col, y, part);
    if (mu.unit_done(jl)) {
      // the block's last unit: add its units' sums in order and store them
      const int64_t n0 = (int64_t)gb * RT * 16;
      for (int i = lane; i < RT * 16 * M; i += kWave) {
        const int r = i / M, t = i - r * M;
        float v = part.v[sl * UMAX][r][t];
        for (int w = 1; w < ups; ++w) v += part.v[sl * UMAX + w][r][t];
        const int64_t row = n0 + r;
        if (row < a.n) {
          if (a.y32) *gmem(a.y32 + ((int64_t)t * a.n + row)) = v;
          if (a.y16) *gmem(a.y16 + ((int64_t)t * a.n + row)) = f32_to_bf16(v);
        }
      }
      mu.release(jl);
    }
    jl = jn;
    u = un;
    gb = gn;
    have = more;
  }
  wait_vmem_all();
  mu.end_launch();
}

}  // namespace wq
