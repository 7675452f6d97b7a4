// Streaming-read probe for MI355X: what HBM rate an access pattern reaches
// with no arithmetic, to set the int4 / int8 / bf16 decode kernels' rates
// against (bench.py measures those; this measures the memory system alone).
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         bw_probe.hip -o bw_probe && ./bw_probe
//
// Part 1: one launch over 4 GiB, one 16-wave workgroup per CU, with several
// ways of dealing the bytes to waves (the decode step kernel's shapes among
// them).  Part 2: back-to-back launches over buffers of one size each, the
// regime of one launch per matrix.  Rates count the bytes each pattern reads.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));          \
      return 1;                                                               \
    }                                                                         \
  } while (0)

__device__ __forceinline__ u32x4 ldnt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint32_t ldnt4(const uint32_t* p) { return __builtin_nontemporal_load(p); }

// Every pattern keeps 4 loads per lane in flight (the decode kernels keep
// 4-8).  Piece i of a pattern is read only when it lies inside the buffer.

// grid-stride over 16-byte pieces
__global__ __launch_bounds__(1024) void grid_stride(const u32x4* __restrict__ b, size_t n16, uint32_t* out) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i + u * stride < n16 ? ldnt(b + i + u * stride) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][u];
  }
  if (acc == 0x12345678u) out[0] = acc;
}

// each workgroup one contiguous range; its waves take adjacent 1 KiB pieces
__global__ __launch_bounds__(1024) void wg_range_adjacent(const u32x4* __restrict__ b, size_t n16, uint32_t* out) {
  uint32_t acc = 0;
  const size_t per = (n16 / gridDim.x) & ~(size_t)255;
  const u32x4* base = b + (size_t)blockIdx.x * per;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  const size_t step = (size_t)waves * 64;
  for (size_t p = (size_t)wave * 64; p < per; p += 4 * step) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = p + u * step < per ? ldnt(base + p + u * step + lane) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][u];
  }
  if (acc == 0x12345678u) out[0] = acc;
}

// each wave one contiguous sub-range of its workgroup's range
__global__ __launch_bounds__(1024) void wave_subrange(const u32x4* __restrict__ b, size_t n16, uint32_t* out) {
  uint32_t acc = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  const size_t per = (n16 / ((size_t)gridDim.x * waves)) & ~(size_t)255;
  const u32x4* base = b + ((size_t)blockIdx.x * waves + wave) * per;
  for (size_t p = 0; p < per; p += 256) {   // per is a multiple of 256
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = ldnt(base + p + 64 * u + lane);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][u];
  }
  if (acc == 0x12345678u) out[0] = acc;
}

// the int4 decode step's shape: rows of 2 KiB of codes + 512 B of (scale,
// zero) words; waves claim batches of 2 consecutive rows from an LDS counter
// and read per row 2 x 1 KiB of codes (16 B per lane) and 2 x 256 B of words
// (4 B per lane).  SEP: words in their own region (the library's format);
// otherwise each 1 KiB of codes is followed by its 256 B of words.
template <bool SEP>
__global__ __launch_bounds__(1024) void int4_rows(const uint8_t* __restrict__ buf, size_t rows, uint32_t* out) {
  __shared__ int ctr;
  uint32_t acc = 0;
  const int lane = threadIdx.x & 63;
  const size_t per_wg = rows / gridDim.x / 2 * 2;
  const size_t r0 = (size_t)blockIdx.x * per_wg;
  if (threadIdx.x == 0) ctr = 0;
  __syncthreads();
  for (;;) {
    int bidx = 0;
    if (lane == 0) bidx = atomicAdd(&ctr, 1);
    bidx = __builtin_amdgcn_readfirstlane(bidx);
    if ((size_t)bidx * 2 >= per_wg) break;
    const size_t r = r0 + (size_t)bidx * 2;
    u32x4 c[2][2];
    uint32_t w[2][2];
    for (int u = 0; u < 2; ++u)
      for (int j = 0; j < 2; ++j) {
        const size_t row = r + u;
        if (SEP) {
          c[u][j] = ldnt(reinterpret_cast<const u32x4*>(buf + row * 2048 + (size_t)j * 1024) + lane);
          w[u][j] = ldnt4(reinterpret_cast<const uint32_t*>(buf + rows * 2048 + row * 512 + (size_t)j * 256) + lane);
        } else {
          const uint8_t* base = buf + row * 2560 + (size_t)j * 1280;
          c[u][j] = ldnt(reinterpret_cast<const u32x4*>(base) + lane);
          w[u][j] = ldnt4(reinterpret_cast<const uint32_t*>(base + 1024) + lane);
        }
      }
    for (int u = 0; u < 2; ++u)
      for (int j = 0; j < 2; ++j) acc ^= c[u][j][0] ^ c[u][j][3] ^ w[u][j];
  }
  if (acc == 0x12345678u) out[0] = acc;
}

// the matrix-core kernels' shape: rows of 8 KiB (int8, k = 8192); waves
// claim batches of BR rows and stream them in passes of 8 KiB per wave (BPP
// bytes of each row, 8 loads of 16 B per lane).  One load instruction spans
// RPI rows x 1024 / RPI contiguous bytes: lane l reads row l % RPI of its
// group at byte 16 (l / RPI) of the span.  RPI = 16 is the MFMA tile
// layout (lane l supplies row l % 16); RPI = 1 reads 1 KiB of one row.
template <int BR, int BPP, int RPI>
__global__ __launch_bounds__(1024) void tile_rows(const uint8_t* __restrict__ buf, size_t rows, uint32_t* out) {
  static_assert(BR * BPP == 8192 && BPP % (1024 / RPI) == 0 && BR % RPI == 0, "8 KiB per pass");
  constexpr size_t RB = 8192;
  constexpr int SPAN = 1024 / RPI, PIECES = BPP / SPAN;
  __shared__ int ctr;
  uint32_t acc = 0;
  const int lane = threadIdx.x & 63;
  const size_t per_wg = rows / gridDim.x / BR * BR;
  const size_t r0 = (size_t)blockIdx.x * per_wg;
  if (threadIdx.x == 0) ctr = 0;
  __syncthreads();
  for (;;) {
    int bidx = 0;
    if (lane == 0) bidx = atomicAdd(&ctr, 1);
    bidx = __builtin_amdgcn_readfirstlane(bidx);
    if ((size_t)bidx * BR >= per_wg) break;
    const uint8_t* base = buf + (r0 + (size_t)bidx * BR) * RB;
    for (size_t pass = 0; pass < RB / BPP; ++pass) {
      u32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int g = i / PIECES, q = i % PIECES;
        const size_t row = (size_t)g * RPI + (size_t)(lane % RPI);
        const size_t byte = pass * BPP + (size_t)q * SPAN + (size_t)(lane / RPI) * 16;
        v[i] = ldnt(reinterpret_cast<const u32x4*>(base + row * RB + byte));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc ^= v[i][i & 3];
    }
  }
  if (acc == 0x12345678u) out[0] = acc;
}

int main() {
  const size_t bytes = (size_t)4 << 30, n16 = bytes / 16;
  u32x4* b;
  uint32_t* out;
  CHECK(hipMalloc(&b, bytes));
  CHECK(hipMalloc(&out, 64));
  CHECK(hipMemset(b, 1, bytes));
  int cus = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const size_t rows = bytes / 2560, rows_used = rows / cus / 2 * 2 * cus;
  printf("part 1: one launch over 4 GiB, %d workgroups x 16 waves (best of 5)\n", cus);
  const char* names[5] = {"grid-stride 16 B pieces", "workgroup ranges, waves on adjacent 1 KiB",
                          "workgroup ranges, one sub-range per wave", "int4 step rows, words in own region",
                          "int4 step rows, words after their codes"};
  for (int k = 0; k < 5; ++k) {
    float best = 1e30f;
    for (int it = 0; it < 5; ++it) {
      CHECK(hipEventRecord(e0));
      if (k == 0) grid_stride<<<cus, 1024>>>(b, n16, out);
      if (k == 1) wg_range_adjacent<<<cus, 1024>>>(b, n16, out);
      if (k == 2) wave_subrange<<<cus, 1024>>>(b, n16, out);
      if (k == 3) int4_rows<true><<<cus, 1024>>>(reinterpret_cast<const uint8_t*>(b), rows, out);
      if (k == 4) int4_rows<false><<<cus, 1024>>>(reinterpret_cast<const uint8_t*>(b), rows, out);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      if (ms < best) best = ms;
    }
    const double moved = k >= 3 ? (double)rows_used * 2560 : (double)bytes;
    printf("  %-44s %.3f ms  %7.1f GB/s\n", names[k], best, moved / best / 1e6);
  }
  printf("part 1b: tile patterns over 4 GiB of 8 KiB rows, %d workgroups x 16 waves (best of 5)\n", cus);
  const size_t trows = bytes / 8192;
  const char* tnames[7] = {"64 rows/batch, 128 B/row/pass, 16 rows/load", "64 rows/batch, 128 B/row/pass,  8 rows/load",
                           "32 rows/batch, 256 B/row/pass, 16 rows/load", "32 rows/batch, 256 B/row/pass,  4 rows/load",
                           "16 rows/batch, 512 B/row/pass, 16 rows/load", "16 rows/batch, 512 B/row/pass,  2 rows/load",
                           " 8 rows/batch,  1 KiB/row/pass, 1 row/load"};
  for (int k = 0; k < 7; ++k) {
    float best = 1e30f;
    for (int it = 0; it < 5; ++it) {
      CHECK(hipEventRecord(e0));
      const uint8_t* bb = reinterpret_cast<const uint8_t*>(b);
      if (k == 0) tile_rows<64, 128, 16><<<cus, 1024>>>(bb, trows, out);
      if (k == 1) tile_rows<64, 128, 8><<<cus, 1024>>>(bb, trows, out);
      if (k == 2) tile_rows<32, 256, 16><<<cus, 1024>>>(bb, trows, out);
      if (k == 3) tile_rows<32, 256, 4><<<cus, 1024>>>(bb, trows, out);
      if (k == 4) tile_rows<16, 512, 16><<<cus, 1024>>>(bb, trows, out);
      if (k == 5) tile_rows<16, 512, 2><<<cus, 1024>>>(bb, trows, out);
      if (k == 6) tile_rows<8, 1024, 1><<<cus, 1024>>>(bb, trows, out);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      if (ms < best) best = ms;
    }
    const size_t br = k < 2 ? 64 : (k < 4 ? 32 : (k < 6 ? 16 : 8));
    const double moved = (double)(trows / cus / br * br * cus) * 8192;
    printf("  %-44s %.3f ms  %7.1f GB/s\n", tnames[k], best, moved / best / 1e6);
  }
  printf("part 2: back-to-back launches over one buffer size (grid-stride, %d x 1024 threads)\n", cus * 2);
  for (size_t mb = 8; mb <= 512; mb *= 2) {
    const size_t nb = mb << 20, launches = bytes / nb;
    CHECK(hipEventRecord(e0));
    for (size_t i = 0; i < launches; ++i)
      grid_stride<<<cus * 2, 1024>>>(reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(b) + i * nb), nb / 16, out);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    printf("  %4zu MB x %4zu launches: %7.1f GB/s (%.2f us per launch)\n", mb, launches, (double)bytes / ms / 1e6,
           ms * 1e3 / launches);
  }
  CHECK(hipFree(b));
  CHECK(hipFree(out));
  return 0;
}
