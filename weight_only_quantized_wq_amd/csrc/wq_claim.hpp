// Work claimed while a one-matrix launch runs (the single-matrix verify
// kernels of wq_verify.hpp and wq_step_i8mt.hpp).
//
// The matrix is cut into blocks of rows and each block into units (a
// stretch of the row's inputs).  The waves of a workgroup claim units in
// order from an LDS counter, so a slower wave simply takes fewer; each
// unit's sums go to their own LDS slot, and the wave that finishes a block's
// last unit adds the slots in unit order, so a result does not depend on
// which wave streamed what.  Slots come in a ring of R blocks: a unit of
// block j waits until block j - R has been added up.
//
// A workgroup's first two blocks are its own (blockIdx.x and blockIdx.x +
// gridDim.x); halfway through each block from its second on, the block
// after it is claimed from the launch's MatrixClaim, so faster workgroups
// take more blocks (at most `cap` each).  The claim is made only once the
// current block's number is known: one workgroup's claims then land in
// order, its blocks increase, and the first block past the matrix ends its
// work (two claims in flight at once could land swapped and strand a
// block).  The launch's last workgroup to finish leaves its MatrixClaim
// zeroed for the next launch that takes it.
#pragma once

#include <stdint.h>

#include "wq_step_shared.hpp"

namespace wq {

// Blocks one workgroup takes at most.
constexpr int kMatrixMaxLocal = 64;

struct MatrixClaim {
  int32_t next;
  int32_t done;
};

// Waits for an LDS word written by another wave of the workgroup: until it
// differs from `v` (!until_equal) or equals it.  The waits of the claiming
// kernels end once older work of the workgroup has finished; the bound turns
// a broken invariant into wrong results instead of a wave that never ends.
__device__ __forceinline__ int lds_wait(const int* p, int v, bool until_equal) {
  int x = 0;
  for (int spin = 0; spin < (1 << 22); ++spin) {
    x = __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
    if ((x == v) == until_equal) break;
    __builtin_amdgcn_s_sleep(2);
  }
  return x;
}

template <int R>
struct MatrixUnitLds {
  int gblk[kMatrixMaxLocal];   // global block of local block j; -1 until claimed
  int uctr;                    // units claimed
  int cnt[R];                  // units of the slot's block finished
  int freed[R];                // last local block added up out of the slot
};

template <int R>
struct MatrixUnits {
  MatrixUnitLds<R>& s;
  MatrixClaim* claim;
  int ups;    // units per block
  int cap;    // blocks per workgroup at most (<= kMatrixMaxLocal)
  int nb;     // blocks of the matrix
  int lane;

  // Wave 0, before the workgroup's first barrier: units [0, first) are
  // taken without a claim (unit w by wave w).
  __device__ __forceinline__ void init(int wave, int first) {
    if (wave != 0) return;
    for (int j = lane; j < kMatrixMaxLocal; j += kWave)
      s.gblk[j] = j == 0 ? (int)blockIdx.x : (j == 1 ? (int)(blockIdx.x + gridDim.x) : -1);
    if (lane == 0) {
      s.uctr = first;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        s.cnt[r] = 0;
        s.freed[r] = r - R;
      }
    }
  }

  // Unit i: local block jl, unit u of it, global block gb.  False when the
  // unit lies past the work.
  __device__ __forceinline__ bool resolve(int i, int& jl, int& u, int& gb) {
    jl = i / ups;
    u = i - jl * ups;
    if (jl >= cap) return false;
    int v = 0;
    if (lane == 0) {
      v = lds_wait(&s.gblk[jl], -1, false);
      if (jl >= 1 && u == ups / 2 && jl + 1 < cap) {
        const int nx = v >= 0 && v < nb ? 2 * (int)gridDim.x + atomicAdd(&claim->next, 1) : nb;
        __hip_atomic_store(&s.gblk[jl + 1], nx, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    gb = __builtin_amdgcn_readfirstlane(v);
    return gb >= 0 && gb < nb;
  }
  __device__ __forceinline__ bool claim_next(int& jl, int& u, int& gb) {
    return resolve(claim_batch(&s.uctr, lane), jl, u, gb);
  }

  // Before a unit of block jl writes its slot: the slot's previous block
  // has been added up.
  __device__ __forceinline__ void wait_slot(int jl) {
    if (lane == 0) lds_wait(&s.freed[jl % R], jl - R, true);
    __builtin_amdgcn_wave_barrier();
  }
  // After the unit's sums are in its slot: true for the block's last unit,
  // whose wave then adds the slots up and calls release.
  __device__ __forceinline__ bool unit_done(int jl) {
    __builtin_amdgcn_wave_barrier();
    int done = 0;
    if (lane == 0) done = __hip_atomic_fetch_add(&s.cnt[jl % R], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    done = __builtin_amdgcn_readfirstlane(done);
    __builtin_amdgcn_wave_barrier();
    return done == ups - 1;
  }
  __device__ __forceinline__ void release(int jl) {
    __builtin_amdgcn_wave_barrier();
    if (lane == 0) {
      __hip_atomic_store(&s.cnt[jl % R], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_store(&s.freed[jl % R], jl, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }

  // Every thread, once its wave has no more work: the launch's last
  // workgroup zeroes the MatrixClaim.
  __device__ __forceinline__ void end_launch() {
    __syncthreads();
    if (threadIdx.x == 0 &&
        __hip_atomic_fetch_add(&claim->done, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1) {
      __hip_atomic_store(&claim->next, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&claim->done, 0, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
};

}  // namespace wq
