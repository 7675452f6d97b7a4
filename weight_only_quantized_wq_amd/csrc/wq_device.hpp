// Device helpers shared by the libwq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// bf16 <-> fp32

__device__ __forceinline__ float bf16lo_to_f32(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t pair) {
  return __uint_as_float(pair & 0xFFFF0000u);
}

// fp32 -> bf16, round to nearest, ties to even.  Adding 0x7FFF plus the kept
// part's lowest bit and truncating rounds the dropped half correctly; a
// carry into the exponent is the correctly rounded result.  NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------------------
// Global-memory views of device pointers.  Pointers read from descriptors in
// memory are generic, and generic accesses compile to FLAT instructions.  A
// FLAT access may target LDS, so while one is outstanding the compiler's
// wait insertion can no longer count vector loads separately and waits for
// ALL of them (vmcnt(0)) before any loaded value is used -- which drains a
// software prefetch pipeline at every such point.  Every pointer the kernels
// dereference outside LDS is global memory, and goes through gmem().

template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gmem(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gmem(const T* p) {
  return (const __attribute__((address_space(1))) T*)p;
}

// Waits for every outstanding vector-memory access.  A loop that ends with a
// prefetch still in flight hands it to whatever code follows, and the wait
// bookkeeping of the next loop, merging that path, may then drain all loads
// in every iteration; draining once where the loop ends is cheaper.
// (s_waitcnt with vmcnt = 0, expcnt and lgkmcnt at their "no wait" maxima.)
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------
// Streaming loads: weights are read exactly once per product, so they are
// fetched with the nontemporal hint and do not displace x or other data.

__device__ __forceinline__ u32x4 load_stream16(const void* p) {
  return __builtin_nontemporal_load(gmem(reinterpret_cast<const u32x4*>(p)));
}
__device__ __forceinline__ u32x4 load16(const void* p) { return *gmem(reinterpret_cast<const u32x4*>(p)); }
__device__ __forceinline__ uint32_t load_stream4(const void* p) {
  return __builtin_nontemporal_load(gmem(reinterpret_cast<const uint32_t*>(p)));
}

// Buffer resource over [base, base + bytes): loads at offsets past `bytes`
// return zero instead of touching memory, so ragged rows and chunks need no
// branches.  Dword 3 selects 32-bit data format (raw, untyped loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// cache policy 2 = nontemporal (streamed once)
__device__ __forceinline__ u32x4 buffer_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
}
__device__ __forceinline__ uint32_t buffer_load4_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 2);
}
// default cache policy (data that other waves read again, e.g. activations)
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// A constant held in a VGPR.  gfx9 VOP3 instructions cannot take two
// literal/SGPR operands, so a mask used with a second constant (as in
// v_and_or_b32) must live in a vector register for the three-operand form.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  uint32_t v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(c));
  return v;
}

// ---------------------------------------------------------------------------
// Packed bf16 dot: a.lo*b.lo + a.hi*b.hi + c in fp32 (v_dot2_f32_bf16).

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

// ---------------------------------------------------------------------------
// Wave-wide sum with DPP.  Quad butterflies, then the half-row and row
// mirrors make every lane hold its 16-lane row's sum; two row broadcasts
// fold rows 0+1 and 2+3 and then the halves; lane 63 ends with the total,
// which is read back as a wave-uniform value.  The order of additions is
// fixed, so the result is deterministic.

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);          // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);          // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);         // row_half_mirror
  v += dpp_f<0x140>(v);         // row_mirror
  v += dpp_f<0x142, 0xA>(v);    // row_bcast15 into rows 1 and 3
  v += dpp_f<0x143, 0xC>(v);    // row_bcast31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Wave-wide maximum of non-negative values (rows the broadcasts skip see 0).
__device__ __forceinline__ float wave_max_nonneg(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  v = fmaxf(v, dpp_f<0x142, 0xA>(v));
  v = fmaxf(v, dpp_f<0x143, 0xC>(v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// A value the caller knows to be equal in every lane, as a wave-uniform
// (scalar) value: descriptors and buffer resources built from it stay in
// scalar registers instead of becoming per-lane loops.
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

}  // namespace wq
