// Weight formats as seen by the streaming matvec kernels.
//
// Every format is consumed in 16-byte chunks: one nontemporal dwordx4 load
// per lane per chunk, 64 consecutive chunks of one row per wave-wide load.
// A lane keeps the activations of the chunks it owns in registers for the
// whole kernel (they are the same for every row), so the hot loop only
// streams weights and does register arithmetic.
//
//   bf16   8 weights / chunk: 4 x v_dot2_f32_bf16 against bf16 x pairs.
//   int8  16 weights / chunk: code bytes XOR 0x80 become u = q + 128 in
//         [1, 255]; v_cvt_f32_ubyte{0..3} + fp32 FMA; the lane subtracts
//         128 * (sum of its x) once per row, and the row scale is applied
//         after the reduction.
//   int4  32 weights / chunk = exactly one group: each nibble is OR-ed into
//         the mantissa of bf16 128.0 (0x4300), giving the exact bf16 value
//         128 + q, two per 32-bit word, fed to v_dot2_f32_bf16.  With
//         A = sum (128 + q) x over the group and X = sum x over the group,
//         the group contributes s * A + (z - 128 s) * X = sum (z + q s) x.
//         (w & 0x000F000F) pairs the codes of k and k + 4 inside an 8-code
//         word, so the activation pairs are pre-permuted once per lane
//         instead of repacking any weight.
#pragma once

#include "wq_device.hpp"

namespace wq {

// ---------------------------------------------------------------------------
struct FmtBf16 {
  static constexpr int kWeightsPerChunk = 8;
  static constexpr bool kGroupAux = false;
  static constexpr bool kRowScale = false;
  static constexpr bool kLaneBias = false;
  struct X {
    uint32_t p[4];
  };

  __device__ static X load_x(const uint16_t* x, int c, bool ok) {
    X r;
    u32x4 v = ok ? load16(x + 8 * (int64_t)c) : u32x4{0, 0, 0, 0};
    r.p[0] = v[0];
    r.p[1] = v[1];
    r.p[2] = v[2];
    r.p[3] = v[3];
    return r;
  }
  __device__ static float lane_bias(const X&) { return 0.0f; }

  // Activations staged in LDS for a whole workgroup: 4 words per chunk (the
  // 8 bf16 values as loaded), chunk c at word 4 c; chunks at or past
  // `chunks` are zero.
  static constexpr int kLdsWordsPerChunk = 4;
  __device__ static void stage(const uint16_t* x, int chunks, int c, uint32_t* xs, int) {
    const X r = load_x(x, c, c < chunks);
    *reinterpret_cast<u32x4*>(xs + 4 * c) = u32x4{r.p[0], r.p[1], r.p[2], r.p[3]};
  }
  __device__ static X lds_x(const uint32_t* xs, int, int c) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xs + 4 * c);
    return X{{v[0], v[1], v[2], v[3]}};
  }

  struct K {};
  __device__ static K consts() { return K{}; }
  // decoded chunk: the bf16 pairs as loaded
  struct D {
    uint32_t p[4];
  };
  __device__ static void decode(const u32x4& w, D& d, const K&) {
    d.p[0] = w[0];
    d.p[1] = w[1];
    d.p[2] = w[2];
    d.p[3] = w[3];
  }
  __device__ static float dot(const D& d, uint32_t, const X& x, float acc) {
    acc = dot2_bf16(d.p[0], x.p[0], acc);
    acc = dot2_bf16(d.p[1], x.p[1], acc);
    acc = dot2_bf16(d.p[2], x.p[2], acc);
    acc = dot2_bf16(d.p[3], x.p[3], acc);
    return acc;
  }
};

// ---------------------------------------------------------------------------
struct FmtInt8 {
  static constexpr int kWeightsPerChunk = 16;
  static constexpr bool kGroupAux = false;
  static constexpr bool kRowScale = true;
  static constexpr bool kLaneBias = false;
  struct X {
    float v[16];
  };

  // bf16 activations
  __device__ static X load_x(const uint16_t* x, int c, bool ok) {
    X r;
    u32x4 a = ok ? load16(x + 16 * (int64_t)c) : u32x4{0, 0, 0, 0};
    u32x4 b = ok ? load16(x + 16 * (int64_t)c + 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      r.v[2 * t] = bf16lo_to_f32(a[t]);
      r.v[2 * t + 1] = bf16hi_to_f32(a[t]);
      r.v[8 + 2 * t] = bf16lo_to_f32(b[t]);
      r.v[8 + 2 * t + 1] = bf16hi_to_f32(b[t]);
    }
    return r;
  }
  // fp32 activations (the MoE down projection consumes the fp32 SwiGLU output)
  __device__ static X load_x(const float* x, int c, bool ok) {
    X r;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 a = ok ? load16(x + 16 * (int64_t)c + 4 * t) : u32x4{0, 0, 0, 0};
      r.v[4 * t] = __uint_as_float(a[0]);
      r.v[4 * t + 1] = __uint_as_float(a[1]);
      r.v[4 * t + 2] = __uint_as_float(a[2]);
      r.v[4 * t + 3] = __uint_as_float(a[3]);
    }
    return r;
  }
  __device__ static float lane_bias(const X&) { return 0.0f; }

  // Activations staged in LDS for a whole workgroup: 17 words per chunk over
  // `cmax` chunks, four 16-byte planes of fp32 values (plane h of chunk c at
  // word 4 * (h * cmax + c)) followed by a bias word (word 16 * cmax + c;
  // zero: the codes decode signed, so no per-row correction is needed).
  // Chunks at or past `chunks` are zero.
  static constexpr int kLdsWordsPerChunk = 17;
  template <class T>
  __device__ static void stage(const T* x, int chunks, int c, uint32_t* xs, int cmax) {
    const X r = load_x(x, c, c < chunks);
#pragma unroll
    for (int h = 0; h < 4; ++h)
      *reinterpret_cast<u32x4*>(xs + 4 * (h * cmax + c)) =
          u32x4{__float_as_uint(r.v[4 * h]), __float_as_uint(r.v[4 * h + 1]), __float_as_uint(r.v[4 * h + 2]),
                __float_as_uint(r.v[4 * h + 3])};
    xs[16 * cmax + c] = __float_as_uint(lane_bias(r));
  }
  __device__ static X lds_x(const uint32_t* xs, int cmax, int c) {
    X r;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(xs + 4 * (h * cmax + c));
      r.v[4 * h] = __uint_as_float(v[0]);
      r.v[4 * h + 1] = __uint_as_float(v[1]);
      r.v[4 * h + 2] = __uint_as_float(v[2]);
      r.v[4 * h + 3] = __uint_as_float(v[3]);
    }
    return r;
  }
  __device__ static float lds_bias(const uint32_t* xs, int cmax, int c) { return __uint_as_float(xs[16 * cmax + c]); }

  struct K {};
  __device__ static K consts() { return K{}; }
  // decoded chunk: the codes q as fp32, one per weight (a sign-extending
  // byte conversion each: v_cvt_f32_i32 with a sign-extended byte operand)
  struct D {
    float u[16];
  };
  __device__ static void decode(const u32x4& w, D& d, const K&) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      d.u[4 * t] = (float)(int8_t)(w[t]);
      d.u[4 * t + 1] = (float)(int8_t)(w[t] >> 8);
      d.u[4 * t + 2] = (float)(int8_t)(w[t] >> 16);
      d.u[4 * t + 3] = (float)(int8_t)(w[t] >> 24);
    }
  }
  __device__ static float dot(const D& d, uint32_t, const X& x, float acc) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = fmaf(d.u[i], x.v[i], acc);
    return acc;
  }
};

// ---------------------------------------------------------------------------
struct FmtInt4 {
  static constexpr int kWeightsPerChunk = 32;
  static constexpr bool kGroupAux = true;   // one (scale, zero) word per chunk
  static constexpr bool kRowScale = false;
  static constexpr bool kLaneBias = false;
  static constexpr uint32_t kMagic = 0x43004300u;   // bf16 128.0 in both halves
  struct X {
    uint32_t p[16];   // p[4i + j] = (x[8i + j], x[8i + j + 4]) as a bf16 pair
    float gsum;       // sum of the group's 32 activations
  };

  __device__ static X load_x(const uint16_t* x, int c, bool ok) {
    u32x4 v[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) v[h] = ok ? load16(x + 32 * (int64_t)c + 8 * h) : u32x4{0, 0, 0, 0};
    return from_words(v);
  }
  // The chunk's 32 activations as loaded (16 words, v[h][j] = word 4 h + j)
  // in the layout above, with their sum.
  __device__ static X from_words(const u32x4 (&v)[4]) {
    X r;
    uint32_t wd[16];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      wd[4 * h] = v[h][0];
      wd[4 * h + 1] = v[h][1];
      wd[4 * h + 2] = v[h][2];
      wd[4 * h + 3] = v[h][3];
    }
    // word t of x holds (x[2t], x[2t+1]); an 8-code weight word i spans x
    // words 4i .. 4i+3.
    float gs = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t a = wd[4 * i], b = wd[4 * i + 1], c2 = wd[4 * i + 2], d = wd[4 * i + 3];
      r.p[4 * i + 0] = (a & 0xFFFFu) | (c2 << 16);          // x[8i],   x[8i+4]
      r.p[4 * i + 1] = (a >> 16) | (c2 & 0xFFFF0000u);      // x[8i+1], x[8i+5]
      r.p[4 * i + 2] = (b & 0xFFFFu) | (d << 16);           // x[8i+2], x[8i+6]
      r.p[4 * i + 3] = (b >> 16) | (d & 0xFFFF0000u);       // x[8i+3], x[8i+7]
      gs = dot2_bf16(a, 0x3F803F80u, gs);
      gs = dot2_bf16(b, 0x3F803F80u, gs);
      gs = dot2_bf16(c2, 0x3F803F80u, gs);
      gs = dot2_bf16(d, 0x3F803F80u, gs);
    }
    r.gsum = gs;
    return r;
  }
  __device__ static float lane_bias(const X&) { return 0.0f; }

  // Activations staged in LDS for a whole workgroup (decode-step kernel):
  // 17 words per chunk, laid out over `cmax` chunks as four 16-byte planes
  // (plane h of chunk c at word 4 * (h * cmax + c), so consecutive lanes read
  // consecutive 16-byte slots) followed by the group sums (word 16 * cmax + c).
  static constexpr int kLdsWordsPerChunk = 17;
  __device__ static void stage(const uint16_t* x, int chunks, int c, uint32_t* xs, int cmax) {
    const X r = load_x(x, c, c < chunks);
#pragma unroll
    for (int h = 0; h < 4; ++h)
      *reinterpret_cast<u32x4*>(xs + 4 * (h * cmax + c)) = u32x4{r.p[4 * h], r.p[4 * h + 1], r.p[4 * h + 2],
                                                                 r.p[4 * h + 3]};
    xs[16 * cmax + c] = __float_as_uint(r.gsum);
  }
  __device__ static X lds_x(const uint32_t* xs, int cmax, int c) {
    X r;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(xs + 4 * (h * cmax + c));
      r.p[4 * h] = v[0];
      r.p[4 * h + 1] = v[1];
      r.p[4 * h + 2] = v[2];
      r.p[4 * h + 3] = v[3];
    }
    r.gsum = __uint_as_float(xs[16 * cmax + c]);
    return r;
  }

  // the nibble mask sits in a VGPR so that each pair decodes with one
  // v_and_or_b32 (mask, then OR the bf16 128.0 exponent pattern)
  struct K {
    uint32_t mask;
  };
  __device__ static K consts() { return K{vgpr_const(0x000F000Fu)}; }
  // decoded chunk: bf16 pairs (128 + q_k, 128 + q_{k+4})
  struct D {
    uint32_t t[16];
  };
  __device__ static void decode(const u32x4& w, D& d, const K& k) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t v = w[i];
      d.t[4 * i + 0] = (v & k.mask) | kMagic;
      d.t[4 * i + 1] = ((v >> 4) & k.mask) | kMagic;
      d.t[4 * i + 2] = ((v >> 8) & k.mask) | kMagic;
      d.t[4 * i + 3] = ((v >> 12) & k.mask) | kMagic;
    }
  }
  // adds the group's sum_k (z + q_k s) x_k to acc; sz word: low half =
  // scale bits, high half = zero bits
  __device__ static float dot(const D& d, uint32_t sz, const X& x, float acc) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = dot2_bf16(d.t[i], x.p[i], a);
    float s = __uint_as_float(sz << 16);
    float z = __uint_as_float(sz & 0xFFFF0000u);
    acc = fmaf(s, a, acc);
    return fmaf(fmaf(-128.0f, s, z), x.gsum, acc);
  }
};

}  // namespace wq
