/* Host implementation of the seeded bf16 input generator (see dcp_inputs/__init__.py):
 * splitmix64 (Steele, Lea & Flood, OOPSLA 2014) at counter 3c+k, k = 0..2, with
 * c = row * 1024 + col; the twelve 16-bit fields form an Irwin-Hall(12) sum that is
 * centred and scaled to a unit-variance value, then rounded to bf16 (nearest-even).
 * mode 1 ("census") instead writes bit `col` of `row` (1.0 or 0.0) for col < 24, else 0.
 * dcp_synth_host_rows_f64 writes the same bf16 values widened exactly to float64. */
#include <stdint.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t bias = 0x7FFFu + ((v.u >> 16) & 1u);
  return (uint16_t)((v.u + bias) >> 16);
}

static inline uint16_t gen_value(uint64_t key, uint64_t row, uint32_t col, int mode) {
  if (mode == 1) return (col < 24 && ((row >> col) & 1u)) ? (uint16_t)0x3F80 : (uint16_t)0;
  uint64_t c = row * 1024u + col;
  int64_t acc = 0;
  for (uint64_t k = 0; k < 3; ++k) {
    uint64_t d = mix64(key + (3u * c + k + 1u) * GOLDEN);
    acc += (int64_t)(d & 0xFFFF) + (int64_t)((d >> 16) & 0xFFFF) +
           (int64_t)((d >> 32) & 0xFFFF) + (int64_t)(d >> 48);
  }
  float z = (float)(acc - 393210) / 65536.0f;
  return f32_to_bf16_rne(z);
}

int dcp_synth_host_rows(const uint64_t* row_ids, int64_t n, int32_t cols, uint64_t key, int32_t mode,
                        uint16_t* out) {
  if (!row_ids || !out || n < 0 || cols <= 0 || cols > 1024) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    for (int32_t c = 0; c < cols; ++c) out[i * cols + c] = gen_value(key, row_ids[i], (uint32_t)c, mode);
  }
  return 0;
}

static inline double bf16_to_f64(uint16_t b) {
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)b << 16;
  return (double)v.f;
}

int dcp_synth_host_rows_f64(const uint64_t* row_ids, int64_t n, int32_t cols, uint64_t key, int32_t mode,
                            double* out) {
  if (!row_ids || !out || n < 0 || cols <= 0 || cols > 1024) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    for (int32_t c = 0; c < cols; ++c)
      out[i * cols + c] = bf16_to_f64(gen_value(key, row_ids[i], (uint32_t)c, mode));
  }
  return 0;
}
