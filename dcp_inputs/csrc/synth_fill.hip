// Device implementation of the seeded bf16 input generator (same definition as the
// host version in synth_host.c): splitmix64 (Steele, Lea & Flood, OOPSLA 2014) at
// counter 3c+k with c = row * 1024 + col, an Irwin-Hall(12) sum of the twelve 16-bit
// fields, centred and scaled to unit variance, rounded to bf16 (nearest-even).
// mode 1 ("census") writes bit `col` of `row` (1.0 or 0.0) for col < 24, else 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t bias = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + bias) >> 16);
}

__device__ __forceinline__ uint16_t gen_value(uint64_t key, uint64_t row, uint32_t col, int mode) {
  if (mode == 1) return (col < 24 && ((row >> col) & 1u)) ? (uint16_t)0x3F80 : (uint16_t)0;
  uint64_t c = row * 1024u + col;
  int64_t acc = 0;
#pragma unroll
  for (uint64_t k = 0; k < 3; ++k) {
    uint64_t d = mix64(key + (3u * c + k + 1u) * GOLDEN);
    acc += (int64_t)(d & 0xFFFF) + (int64_t)((d >> 16) & 0xFFFF) +
           (int64_t)((d >> 32) & 0xFFFF) + (int64_t)(d >> 48);
  }
  float z = (float)(acc - 393210) / 65536.0f;
  return f32_to_bf16_rne(z);
}

// One thread per (row, pair of columns); rows whose destination index is outside
// [0, dst_num_rows) are skipped.
__global__ void synth_fill_rows_kernel(uint16_t* __restrict__ dst, int64_t dst_num_rows,
                                       const int64_t* __restrict__ dst_rows,
                                       const int64_t* __restrict__ row_ids, int64_t n, int cols,
                                       uint64_t key, int mode) {
  const int half = (cols + 1) / 2;
  const int64_t total = n * half;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    int64_t i = e / half;
    int c = (int)(e - i * half) * 2;
    int64_t r = dst_rows[i];
    if (r < 0 || r >= dst_num_rows) continue;
    uint64_t id = (uint64_t)row_ids[i];
    uint16_t* p = dst + r * cols + c;
    p[0] = gen_value(key, id, (uint32_t)c, mode);
    if (c + 1 < cols) p[1] = gen_value(key, id, (uint32_t)(c + 1), mode);
  }
}

__global__ void synth_fill_value_kernel(uint16_t* __restrict__ dst, int64_t n, uint16_t bits) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x)
    dst[e] = bits;
}

extern "C" int dcp_synth_fill_rows(void* dst, int64_t dst_num_rows, const int64_t* dst_rows,
                                   const int64_t* row_ids, int64_t n, int32_t cols, uint64_t key,
                                   int32_t mode, hipStream_t stream) {
  if (n == 0) return 0;
  if (!dst || !dst_rows || !row_ids || n < 0 || cols <= 0 || cols > 1024 || dst_num_rows < 0)
    return 1;
  const int64_t total = n * ((cols + 1) / 2);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(synth_fill_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (uint16_t*)dst, dst_num_rows, dst_rows, row_ids, n, (int)cols, key, (int)mode);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int dcp_synth_fill_value(void* dst, int64_t n, uint16_t bits, hipStream_t stream) {
  if (n == 0) return 0;
  if (!dst || n < 0) return 1;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(synth_fill_value_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (uint16_t*)dst, n, bits);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
