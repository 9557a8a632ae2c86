// The N-way LSE merge split into the per-rank steps of a multi-GPU DCP group
// (vLLM blog "Efficient Decode Context Parallelism with vLLM for Long Context
// Workloads", Sec. 4.1, "AllGather + ReduceScatter"): after an all-gather of the
// ranks' LSE values every rank knows the global LSE = ln sum_r exp(LSE_r), rescales
// its own partial by exp(LSE_r - LSE) (its share of the softmax mass), and a
// reduce-scatter sums the rescaled partials, each rank keeping a slice of the heads.
// On one GPU the three steps run as three launches over stacked tensors; their
// result equals the fused merge.
#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {

// Global LSE of each (request, head) row from the N gathered LSE_r.
__global__ __launch_bounds__(256) void merge_lse_kernel(const float* __restrict__ lse_parts, int32_t n,
                                                        int64_t rows, float* __restrict__ out) {
  for (int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; row < rows;
       row += (int64_t)gridDim.x * blockDim.x) {
    float mx = -INFINITY;
    for (int r = 0; r < n; ++r) mx = fmaxf(mx, lse_parts[(int64_t)r * rows + row]);
    if (mx == -INFINITY) { out[row] = -INFINITY; continue; }
    float s = 0.f;
    for (int r = 0; r < n; ++r) s += fast_exp2((lse_parts[(int64_t)r * rows + row] - mx) * kLog2e);
    out[row] = mx + fast_log2(s) * kLn2;
  }
}

// One rank's partial scaled by its share exp(LSE_r - LSE); 4 outputs per thread.
template <bool BF16>
__global__ __launch_bounds__(256) void rescale_kernel(const float* __restrict__ o, const float* __restrict__ lse_r,
                                                      const float* __restrict__ lse, int64_t rows,
                                                      int32_t v_dim, void* __restrict__ out) {
  const int quads = v_dim >> 2;
  const int64_t total = rows * quads;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = e / quads;
    const float g = lse[row], l = lse_r[row];
    // a rank without tokens (or a row nobody attended) carries no weight
    const float s = (g == -INFINITY || l == -INFINITY) ? 0.f : fast_exp2((l - g) * kLog2e);
    // written as a select, so that a part without weight gives 0 even where its O holds NaN
    const f32x4 v = s == 0.f ? f32x4{} : ((const f32x4*)o)[e] * s;
    if (BF16) {
      bf16x4 b;
#pragma unroll
      for (int k = 0; k < 4; ++k) b[k] = (__bf16)v[k];
      ((bf16x4*)out)[e] = b;
    } else {
      ((f32x4*)out)[e] = v;
    }
  }
}

// Rank `rank`'s heads [rank * Hs, (rank + 1) * Hs) of the sum over the N stacked
// rescaled partials [N, B, H, v_dim]; out is [B, Hs, v_dim] fp32.
template <bool BF16>
__global__ __launch_bounds__(256) void sum_slice_kernel(const void* __restrict__ parts, int32_t n, int64_t batch,
                                                        int32_t heads, int32_t slice, int32_t rank,
                                                        int32_t v_dim, float* __restrict__ out) {
  const int quads = v_dim >> 2;
  const int64_t total = batch * slice * quads;
  const int64_t part_quads = batch * heads * quads;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = e / quads;  // (b, h') of the slice
    const int qd = (int)(e - row * quads);
    const int64_t b = row / slice;
    const int h = (int)(row - b * slice) + rank * slice;
    const int64_t src = (b * heads + h) * quads + qd;
    f32x4 acc = f32x4{};
    for (int r = 0; r < n; ++r) {
      if (BF16) {
        const bf16x4 v = ((const bf16x4*)parts)[(int64_t)r * part_quads + src];
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] += (float)v[k];
      } else {
        acc += ((const f32x4*)parts)[(int64_t)r * part_quads + src];
      }
    }
    ((f32x4*)out)[e] = acc;
  }
}

static unsigned grid_for(int64_t items) {
  int64_t blocks = (items + 255) / 256;
  return (unsigned)(blocks > (1 << 20) ? (1 << 20) : (blocks < 1 ? 1 : blocks));
}

hipError_t launch_merge_lse(const float* lse_parts, int32_t n, int64_t rows, float* out, hipStream_t s) {
  hipLaunchKernelGGL(merge_lse_kernel, dim3(grid_for(rows)), dim3(256), 0, s, lse_parts, n, rows, out);
  return hipGetLastError();
}

hipError_t launch_rescale(const float* o, const float* lse_r, const float* lse, int64_t rows,
                          int32_t v_dim, bool bf16, void* out, hipStream_t s) {
  const unsigned g = grid_for(rows * (v_dim / 4));
  if (bf16) hipLaunchKernelGGL(rescale_kernel<true>, dim3(g), dim3(256), 0, s, o, lse_r, lse, rows, v_dim, out);
  else hipLaunchKernelGGL(rescale_kernel<false>, dim3(g), dim3(256), 0, s, o, lse_r, lse, rows, v_dim, out);
  return hipGetLastError();
}

hipError_t launch_sum_slice(const void* parts, bool bf16, int32_t n, int64_t batch, int32_t heads,
                            int32_t rank, int32_t v_dim, float* out, hipStream_t s) {
  const int32_t slice = heads / n;
  const unsigned g = grid_for(batch * slice * (v_dim / 4));
  if (bf16)
    hipLaunchKernelGGL(sum_slice_kernel<true>, dim3(g), dim3(256), 0, s, parts, n, batch, heads, slice, rank, v_dim, out);
  else
    hipLaunchKernelGGL(sum_slice_kernel<false>, dim3(g), dim3(256), 0, s, parts, n, batch, heads, slice, rank, v_dim, out);
  return hipGetLastError();
}

}  // namespace dcp
