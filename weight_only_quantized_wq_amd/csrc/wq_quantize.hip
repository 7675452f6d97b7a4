// Offline quantizers: fp32 weights -> int8 per-row / int4 codes (groups of
// 32, 64, 128 or 256 inputs, or one group per row).
//
// Codes are round-half-even of the EXACT real quotient, so the device must
// take the same decision as exact arithmetic even when an fp32 quotient
// lands within rounding of a half-integer.  A candidate code c comes from an
// fp64 quotient; it is then confirmed or moved by exact comparisons of w
// against the decision boundaries z + (c +- 1/2) s:
//   * (c +- 1/2) s is exact in fp64 (a <= 8-bit integer-and-a-half times an
//     8-bit bf16 significand);
//   * w - z is formed with TwoSum, so d + e == w - z exactly; rounding is
//     monotone, hence d > p implies w - z > p, d < p implies w - z < p, and
//     when d == p the sign of (w - z) - p is the sign of e.
// An exact tie goes to the even code.
#include <stdint.h>

#include "wq_device.hpp"
#include "wq_host.hpp"

namespace wq {

// sign((w - z) - p) computed exactly (w, z, p are exact fp64 values)
__device__ __forceinline__ int cmp_diff(double w, double z, double p) {
  double d = w - z;
  double bb = d - w;
  double e = (w - (d - bb)) + (-z - bb);
  if (d > p) return 1;
  if (d < p) return -1;
  return (e > 0.0) - (e < 0.0);
}

// round-half-even of the exact (w - z) / s for s > 0, starting from a
// candidate within a few units of the answer.
__device__ __forceinline__ int rne_code(double w, double z, double s, int c) {
  for (int it = 0; it < 6; ++it) {
    int up = cmp_diff(w, z, ((double)c + 0.5) * s);
    if (up > 0 || (up == 0 && (c & 1))) {
      ++c;
      continue;
    }
    int dn = cmp_diff(w, z, ((double)c - 0.5) * s);
    if (dn < 0 || (dn == 0 && (c & 1))) {
      --c;
      continue;
    }
    break;
  }
  return c;
}

__device__ __forceinline__ int candidate(double w, double z, double s, int lo, int hi) {
  double r = rint((w - z) / s);
  if (!(r >= (double)lo)) r = (double)lo;   // also catches NaN
  if (r > (double)hi) r = (double)hi;
  return (int)r;
}

// ---------------------------------------------------------------------------
// int8: one wave per row.

__global__ __launch_bounds__(256) void quantize_int8_kernel(const float* __restrict__ w, int64_t n, int64_t k,
                                                            int8_t* __restrict__ q, uint16_t* __restrict__ scale) {
  const int lane = lane_id();
  const int64_t waves = (int64_t)gridDim.x * 4;
  const int64_t k4 = k / 4;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < n; r += waves) {
    const float4* row = reinterpret_cast<const float4*>(w + r * k);
    float m = 0.0f;
    for (int64_t i = lane; i < k4; i += kWave) {
      float4 v = row[i];
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    m = wave_max_nonneg(m);
    const uint16_t sb = f32_to_bf16(__fdiv_rn(m, 127.0f));
    const double s = (double)__uint_as_float((uint32_t)sb << 16);
    if (lane == 0) scale[r] = sb;
    uint32_t* qrow = reinterpret_cast<uint32_t*>(q + r * k);
    for (int64_t i = lane; i < k4; i += kWave) {
      float4 v = row[i];
      float e[4] = {v.x, v.y, v.z, v.w};
      uint32_t packed = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        int c = 0;
        if (s > 0.0) {
          double wd = (double)e[t];
          c = rne_code(wd, 0.0, s, candidate(wd, 0.0, s, -200, 200));
          c = c < -127 ? -127 : (c > 127 ? 127 : c);
        }
        packed |= ((uint32_t)(uint8_t)(int8_t)c) << (8 * t);
      }
      qrow[i] = packed;
    }
  }
}

// ---------------------------------------------------------------------------
// int4: shared per-group arithmetic.

// (scale, zero) bf16 bits of a group from its fp32 min and max: z = bf16(min)
// with a zero minimum taken as +0 (min + 0 maps -0 to +0 and nothing else),
// t = fp32(max - z), s = bf16(fp32(t / 15)) if t > 0 else 0.
__device__ __forceinline__ void int4_scale_zero_bits(float mn, float mx, uint16_t& sb, uint16_t& zb) {
  zb = f32_to_bf16(__fadd_rn(mn, 0.0f));
  const float zf = __uint_as_float((uint32_t)zb << 16);
  const float t = __fsub_rn(mx, zf);
  sb = t > 0.0f ? f32_to_bf16(__fdiv_rn(t, 15.0f)) : (uint16_t)0;
}

// Packed codes of 32 consecutive inputs (8 float4 from src): byte j holds
// code 2j in its low nibble and code 2j + 1 in its high nibble.
__device__ __forceinline__ u32x4 int4_code_chunk(const float4* src, double s, double z) {
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 t4 = src[i];
    v[4 * i] = t4.x;
    v[4 * i + 1] = t4.y;
    v[4 * i + 2] = t4.z;
    v[4 * i + 3] = t4.w;
  }
  uint32_t words[4] = {0u, 0u, 0u, 0u};
  if (s > 0.0) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const double wd = (double)v[i];
      int c = rne_code(wd, z, s, candidate(wd, z, s, -64, 64));
      c = c < 0 ? 0 : (c > 15 ? 15 : c);
      words[i >> 3] |= (uint32_t)c << (4 * (i & 7));
    }
  }
  return u32x4{words[0], words[1], words[2], words[3]};
}

// ---------------------------------------------------------------------------
// int4 with groups of G (32, 64, 128, 256): one lane per group of G
// consecutive inputs -- a pass over the group for (min, max), then the codes
// 32 inputs (16 output bytes) at a time.

template <int G>
__global__ __launch_bounds__(256) void quantize_int4_kernel(const float* __restrict__ w, int64_t n, int64_t k,
                                                            uint8_t* __restrict__ qpacked, uint32_t* __restrict__ sz) {
  const int64_t groups_per_row = k / G;
  const int64_t total = n * groups_per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t gidx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gidx < total; gidx += stride) {
    const int64_t r = gidx / groups_per_row;
    const int64_t g = gidx - r * groups_per_row;
    const float4* src = reinterpret_cast<const float4*>(w + r * k + g * G);
    float mn = src[0].x, mx = src[0].x;
    for (int i = 0; i < G / 4; ++i) {
      const float4 t = src[i];
      mn = fminf(fminf(mn, t.x), fminf(t.y, fminf(t.z, t.w)));
      mx = fmaxf(fmaxf(mx, t.x), fmaxf(t.y, fmaxf(t.z, t.w)));
    }
    uint16_t sb, zb;
    int4_scale_zero_bits(mn, mx, sb, zb);
    const double s = (double)__uint_as_float((uint32_t)sb << 16);
    const double z = (double)__uint_as_float((uint32_t)zb << 16);
    for (int c32 = 0; c32 < G / 32; ++c32)
      *reinterpret_cast<u32x4*>(qpacked + r * (k / 2) + g * (G / 2) + 16 * c32) = int4_code_chunk(src + 8 * c32, s, z);
    sz[gidx] = (uint32_t)sb | ((uint32_t)zb << 16);
  }
}

// ---------------------------------------------------------------------------
// int4 with one group per row (per-channel): one wave per row.  The wave
// reduces the row's min and max with a butterfly (every lane ends with both;
// a zero minimum is normalised to +0 afterwards, so the order in which +0 and
// -0 meet does not matter), then lane l codes chunks l, l + 64, ...

__device__ __forceinline__ void wave_min_max(float& mn, float& mx) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
  }
}

__global__ __launch_bounds__(256) void quantize_int4_row_kernel(const float* __restrict__ w, int64_t n, int64_t k,
                                                                uint8_t* __restrict__ qpacked,
                                                                uint32_t* __restrict__ sz) {
  const int lane = lane_id();
  const int64_t waves = (int64_t)gridDim.x * 4;
  const int64_t k4 = k / 4;
  const int64_t chunks = k / 32;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < n; r += waves) {
    const float4* row = reinterpret_cast<const float4*>(w + r * k);
    float mn = __builtin_inff(), mx = -__builtin_inff();
    for (int64_t i = lane; i < k4; i += kWave) {
      const float4 t = row[i];
      mn = fminf(fminf(mn, t.x), fminf(t.y, fminf(t.z, t.w)));
      mx = fmaxf(fmaxf(mx, t.x), fmaxf(t.y, fmaxf(t.z, t.w)));
    }
    wave_min_max(mn, mx);
    uint16_t sb, zb;
    int4_scale_zero_bits(mn, mx, sb, zb);
    const double s = (double)__uint_as_float((uint32_t)sb << 16);
    const double z = (double)__uint_as_float((uint32_t)zb << 16);
    for (int64_t c = lane; c < chunks; c += kWave)
      *reinterpret_cast<u32x4*>(qpacked + r * (k / 2) + 16 * c) = int4_code_chunk(row + 8 * c, s, z);
    if (lane == 0) sz[r] = (uint32_t)sb | ((uint32_t)zb << 16);
  }
}

}  // namespace wq

using namespace wq;

extern "C" int wq_quantize_int8(const float* w, int64_t n, int64_t k, int8_t* q, uint16_t* scale, void* stream) {
  const char* name = "wq_quantize_int8";
  if (!w || !q || !scale) return fail(WQ_ERR_NULL, "%s: w, q and scale must be non-null", name);
  if (n < 0 || k < 0 || k % 4) return fail(WQ_ERR_SHAPE, "%s: need n, k >= 0 and k %% 4 == 0 (n = %lld, k = %lld)", name, (long long)n, (long long)k);
  if (!aligned16(w) || (reinterpret_cast<uintptr_t>(q) & 3u) || (reinterpret_cast<uintptr_t>(scale) & 1u))
    return fail(WQ_ERR_ALIGN, "%s: w must be 16-byte, q 4-byte and scale 2-byte aligned", name);
  if (n == 0) return WQ_OK;
  int rc = check_device();
  if (rc) return rc;
  const int resident = resident_groups(reinterpret_cast<const void*>(quantize_int8_kernel), 256);
  int64_t grid = balanced_grid((n + 3) / 4, resident);
  hipLaunchKernelGGL(quantize_int8_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, w, n, k, q,
                     scale);
  return launch_status(name);
}

template <int G>
static int launch_quantize_int4(const float* w, int64_t n, int64_t k, uint8_t* qpacked, uint16_t* sz,
                                hipStream_t stream, const char* name) {
  const int resident = resident_groups(reinterpret_cast<const void*>(quantize_int4_kernel<G>), 256);
  const int64_t blocks = (n * (k / G) + 255) / 256;
  const int64_t grid = balanced_grid(blocks, resident);
  hipLaunchKernelGGL(quantize_int4_kernel<G>, dim3((unsigned)grid), dim3(256), 0, stream, w, n, k, qpacked,
                     reinterpret_cast<uint32_t*>(sz));
  return launch_status(name);
}

extern "C" int wq_quantize_int4(const float* w, int64_t n, int64_t k, int32_t group, uint8_t* qpacked, uint16_t* sz,
                                void* stream) {
  const char* name = "wq_quantize_int4";
  if (!w || !qpacked || !sz) return fail(WQ_ERR_NULL, "%s: w, qpacked and sz must be non-null", name);
  // one group per row: group == k, k a positive multiple of 32
  const bool per_row = group != 32 && group != 64 && group != 128 && group != 256 && group == k && k > 0;
  if (group != 32 && group != 64 && group != 128 && group != 256 && !per_row)
    return fail(WQ_ERR_SHAPE, "%s: group = %d (need 32, 64, 128, 256 or k = %lld)", name, group, (long long)k);
  const int64_t kmult = per_row ? 32 : group;
  if (n < 0 || k < 0 || k % kmult)
    return fail(WQ_ERR_SHAPE, "%s: need n, k >= 0 and k %% %lld == 0 (n = %lld, k = %lld)", name, (long long)kmult,
                (long long)n, (long long)k);
  if (!aligned16(w) || !aligned16(qpacked) || (reinterpret_cast<uintptr_t>(sz) & 3u))
    return fail(WQ_ERR_ALIGN, "%s: w and qpacked must be 16-byte and sz 4-byte aligned", name);
  if (n == 0 || k == 0) return WQ_OK;
  int rc = check_device();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (per_row) {
    const int resident = resident_groups(reinterpret_cast<const void*>(quantize_int4_row_kernel), 256);
    const int64_t grid = balanced_grid((n + 3) / 4, resident);
    hipLaunchKernelGGL(quantize_int4_row_kernel, dim3((unsigned)grid), dim3(256), 0, st, w, n, k, qpacked,
                       reinterpret_cast<uint32_t*>(sz));
    return launch_status(name);
  }
  switch (group) {
    case 32: return launch_quantize_int4<32>(w, n, k, qpacked, sz, st, name);
    case 64: return launch_quantize_int4<64>(w, n, k, qpacked, sz, st, name);
    case 128: return launch_quantize_int4<128>(w, n, k, qpacked, sz, st, name);
    default: return launch_quantize_int4<256>(w, n, k, qpacked, sz, st, name);
  }
}

extern "C" int wq_quantize_int4g32(const float* w, int64_t n, int64_t k, uint8_t* qpacked, uint16_t* sz,
                                   void* stream) {
  const char* name = "wq_quantize_int4g32";
  if (!w || !qpacked || !sz) return fail(WQ_ERR_NULL, "%s: w, qpacked and sz must be non-null", name);
  if (n < 0 || k < 0 || k % 32)
    return fail(WQ_ERR_SHAPE, "%s: need n, k >= 0 and k %% 32 == 0 (n = %lld, k = %lld)", name, (long long)n, (long long)k);
  if (!aligned16(w) || !aligned16(qpacked) || (reinterpret_cast<uintptr_t>(sz) & 3u))
    return fail(WQ_ERR_ALIGN, "%s: w and qpacked must be 16-byte and sz 4-byte aligned", name);
  if (n == 0 || k == 0) return WQ_OK;
  int rc = check_device();
  if (rc) return rc;
  return launch_quantize_int4<32>(w, n, k, qpacked, sz, (hipStream_t)stream, name);
}
