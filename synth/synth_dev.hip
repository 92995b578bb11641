// Seeded synthetic inputs (device side): the same integer recipe as
// synth_host.c, so that multi-gigabyte weight sets can be drawn straight into
// HBM.  Draws numbers only; holds none of the decode step's arithmetic.
// Every output element i is a pure function of (key, offset + i), which makes
// a device-drawn tensor bit-identical to the host-drawn one.
#include <hip/hip_runtime.h>
#include <stdint.h>

__device__ __forceinline__ uint64_t sm64(uint64_t key, uint64_t i) {
  uint64_t z = key + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float irwin_hall4(uint64_t w, float scale) {
  int32_t s = (int32_t)(w & 0xFFFF) + (int32_t)((w >> 16) & 0xFFFF) +
              (int32_t)((w >> 32) & 0xFFFF) + (int32_t)((w >> 48) & 0xFFFF);
  float f = (float)(s - 131070);
  return __fmul_rn(f, scale);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void k_normal_bf16(uint64_t key, float scale, uint16_t* out, int64_t n, int64_t offset) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = f32_to_bf16_rne(irwin_hall4(sm64(key, (uint64_t)(offset + i)), scale));
}

// A rows x cols matrix whose logical element (r, c) is draw r*cols + c,
// stored in tiles of tr consecutive rows, column-major within a tile:
// element (r, c) sits at ((r / tr) * cols + c) * tr + r % tr.
__global__ void k_normal_bf16_tiles(uint64_t key, float scale, uint16_t* out, int64_t rows, int64_t cols, int64_t tr) {
  const int64_t n = rows * cols, tile = tr * cols;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n; q += stride) {
    const int64_t t = q / tile, w = q % tile;
    const int64_t r = t * tr + w % tr, c = w / tr;
    out[q] = f32_to_bf16_rne(irwin_hall4(sm64(key, (uint64_t)(r * cols + c)), scale));
  }
}

__global__ void k_normal_f32(uint64_t key, float scale, float* out, int64_t n, int64_t offset) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = irwin_hall4(sm64(key, (uint64_t)(offset + i)), scale);
}

__global__ void k_uniform_i32(uint64_t key, int32_t hi, int32_t* out, int64_t n, int64_t offset) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    uint64_t w = sm64(key, (uint64_t)(offset + i));
    out[i] = (int32_t)(((w >> 32) * (uint64_t)(uint32_t)hi) >> 32);
  }
}

__global__ void k_fill_u16(uint16_t v, uint16_t* out, int64_t n) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) out[i] = v;
}

static unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 16384) g = 16384;
  if (g < 1) g = 1;
  return (unsigned)g;
}

extern "C" int synth_dev_normal_bf16(uint64_t key, float scale, void* out, int64_t n, int64_t offset, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_normal_bf16, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, key, scale, (uint16_t*)out, n, offset);
  return (int)hipGetLastError();
}
extern "C" int synth_dev_normal_bf16_tiles(uint64_t key, float scale, void* out, int64_t rows, int64_t cols,
                                           int64_t tile_rows, void* stream) {
  if (rows <= 0 || cols <= 0) return 0;
  if (tile_rows <= 0 || rows % tile_rows) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_normal_bf16_tiles, dim3(grid_for(rows * cols)), dim3(256), 0, (hipStream_t)stream, key, scale,
                     (uint16_t*)out, rows, cols, tile_rows);
  return (int)hipGetLastError();
}
extern "C" int synth_dev_normal_f32(uint64_t key, float scale, void* out, int64_t n, int64_t offset, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_normal_f32, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, key, scale, (float*)out, n, offset);
  return (int)hipGetLastError();
}
extern "C" int synth_dev_uniform_i32(uint64_t key, int32_t hi, void* out, int64_t n, int64_t offset, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_uniform_i32, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, key, hi, (int32_t*)out, n, offset);
  return (int)hipGetLastError();
}
extern "C" int synth_dev_fill_u16(uint16_t v, void* out, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_fill_u16, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, v, (uint16_t*)out, n);
  return (int)hipGetLastError();
}
