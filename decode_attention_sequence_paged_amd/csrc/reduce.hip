// Log-sum-exp merges and shard-map kernels.
//
// The merge rule is the one the vLLM blog "Efficient Decode Context Parallelism
// with vLLM for Long Context Workloads" states in Sec. 4.1 (its all-gather and
// reduce-scatter step): partial outputs over disjoint token sets are reweighted by
// their LSE values (the rescaling online softmax also uses) and summed,
//   LSE = ln sum_i exp(LSE_i),   O = sum_i exp(LSE_i - LSE) O_i.
// It serves twice: inside a rank, to join the pieces of a request that several
// work partitions computed (split-K), and across the N ranks.
#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {

// ------------------------------------------------------------------ split-K reduce
// One block per (request, group of heads, slice of DV / DS output dims).  A head's
// slice is spread over DV/DS/4/QPT threads, each owning QPT quads of 4 consecutive
// floats kQStride apart (so a wave's loads stay contiguous); with PL > 1, PL such
// thread sets ("piece lanes") fold every PL-th piece of the request and are summed
// through LDS at the end.  The pieces' slots and LSEs are first staged in LDS by the
// whole block, a chunk of kThreads pieces at a time with a running maximum, so any
// piece count works.  The host picks PL from the expected pieces per request
// (partitions / batch): 1 for batches of many requests, up to 8 for a single very
// long request, whose 512 outputs per head are then cut into 4 slices so that the
// merge is spread over four times as many blocks (9.0 instead of 10.0 us for the
// 1M-token request).
template <int DV, int PL, int DS = 1, int QPT = 1>
struct SplitCfg {
  static constexpr int kQuads = DV / 4 / DS / QPT;           // threads per head and piece lane
  static constexpr int kTph = kQuads * PL;                   // threads per head
  static constexpr int kThreads = kTph < 256 ? 256 : kTph;
  static constexpr int kHpb = kThreads / kTph;               // heads per block
  static constexpr int kUnroll = 4;
  static_assert(kThreads % kTph == 0 && kThreads <= 1024, "block shape");
};

template <int DV, int PL, int DS = 1, int QPT = 1>
__global__ __launch_bounds__((SplitCfg<DV, PL, DS, QPT>::kThreads)) void split_reduce_kernel(SplitReduceParams p) {
  using C = SplitCfg<DV, PL, DS, QPT>;
  static_assert(PL == 1 || QPT == 1, "quads per thread only without piece lanes");
  constexpr int kQStride = 4 * C::kQuads;  // floats between a thread's quads
  constexpr int kChunk = C::kThreads;  // pieces staged per round
  __shared__ int64_t s_slot[kChunk];
  __shared__ float s_lse[kChunk][C::kHpb];
  __shared__ f32x4 s_acc[PL > 1 ? C::kThreads : 1];
  __shared__ float s_w[PL > 1 ? C::kThreads : 1];

  const int b = blockIdx.x;
  const int head0 = blockIdx.y * C::kHpb;
  const int hd = (int)threadIdx.x / C::kTph;
  const int head = head0 + hd;
  const int t = (int)threadIdx.x % C::kTph;
  const int q = t % C::kQuads;
  const int pl = t / C::kQuads;
  const int H = p.num_heads;
  const bool head_ok = head < H;

  // the request's partition entry, read in one round: first tile, tile count, weighted
  // position, weighted total, and the spans of its first and last tiles
  const int64_t F = p.ws_prefix[b];
  const int64_t n = p.ws_prefix[b + 1] - F;
  const int64_t WP = p.ws_prefix[p.batch + 1 + b];
  const int64_t WT = p.ws_prefix[2 * p.batch + 1];
  const int64_t span_range = p.ws_prefix[2 * p.batch + 2 + b];
  const int col = (int)blockIdx.z * (DV / DS) + 4 * q;
  float* orow = p.out_o + ((int64_t)b * p.out_req_rows + head) * DV + col;
  if (n == 0) {  // no local tokens: the merge's neutral element
    if (head_ok && pl == 0) {
#pragma unroll
      for (int k = 0; k < QPT; ++k) *(f32x4*)(orow + k * kQStride) = f32x4{};
      if (col == 0) p.out_lse[(int64_t)b * p.out_req_rows + head] = -INFINITY;
    }
    return;
  }
  const int64_t P = p.num_parts;
  const bool xw = p.xcd_weighted != 0;
  const int64_t w_lo = span_range >> 32;
  const int64_t w_hi = span_range & 0xFFFFFFFF;
  if (w_lo == w_hi) return;  // computed in one piece by the partial kernel

  float mx = -INFINITY, wsum = 0.f;
  f32x4 acc[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) acc[k] = f32x4{};
  for (int64_t base = w_lo; base <= w_hi; base += kChunk) {
    const int cnt = (int)((w_hi - base + 1) < kChunk ? (w_hi - base + 1) : kChunk);
    __syncthreads();  // the previous round's LDS reads are done
    for (int i = threadIdx.x; i < cnt; i += C::kThreads) {
      const int64_t w = base + i;
      const int64_t x0 = dcp_span_start(w, WT, P, xw);
      // an empty span holds no piece
      const int64_t slot = dcp_span_empty(w, WT, P, xw) ? -1 : dcp_piece_slot(w, w_lo, x0, WP);
      s_slot[i] = slot;
#pragma unroll
      for (int h = 0; h < C::kHpb; ++h)
        s_lse[i][h] = (slot >= 0 && head0 + h < H) ? p.ws_lse[slot * H + head0 + h] * kLog2e : -INFINITY;
    }
    __syncthreads();
    float cm = -INFINITY;
    for (int i = 0; i < cnt; ++i) cm = fmaxf(cm, s_lse[i][hd]);
    const float nm = fmaxf(mx, cm);
    const float rescale = mx == -INFINITY ? 0.f : fast_exp2(mx - nm);
#pragma unroll
    for (int k = 0; k < QPT; ++k) acc[k] *= rescale;
    wsum *= rescale;
    mx = nm;
    if (head_ok) {
      for (int i0 = pl; i0 < cnt; i0 += PL * C::kUnroll) {
        f32x4 v[C::kUnroll][QPT];
        float wt[C::kUnroll];
#pragma unroll
        for (int u = 0; u < C::kUnroll; ++u) {
          const int i = i0 + u * PL;
          const int64_t slot = i < cnt ? s_slot[i] : -1;
          // empty pieces (a causally masked row) carry no weight
          const float l = i < cnt ? s_lse[i][hd] : -INFINITY;
          wt[u] = slot >= 0 && l != -INFINITY ? fast_exp2(l - mx) : 0.f;
#pragma unroll
          for (int k = 0; k < QPT; ++k)
            v[u][k] = slot >= 0 ? *(const f32x4*)(p.ws_o + (slot * H + head) * DV + col + k * kQStride) : f32x4{};
        }
#pragma unroll
        for (int u = 0; u < C::kUnroll; ++u) {
          wsum += wt[u];
#pragma unroll
          for (int k = 0; k < QPT; ++k) acc[k] += wt[u] * v[u][k];
        }
      }
    }
  }
  if constexpr (PL > 1) {  // every piece lane used the same maximum: plain sums
    s_acc[threadIdx.x] = acc[0];
    s_w[threadIdx.x] = wsum;
    __syncthreads();
    if (pl != 0) return;
    const int base = hd * C::kTph + q;
#pragma unroll
    for (int j = 1; j < PL; ++j) {
      acc[0] += s_acc[base + j * C::kQuads];
      wsum += s_w[base + j * C::kQuads];
    }
  }
  if (!head_ok) return;
  // a row no piece saw a token for: the merge's neutral element
#pragma unroll
  for (int k = 0; k < QPT; ++k) *(f32x4*)(orow + k * kQStride) = wsum > 0.f ? acc[k] * (1.0f / wsum) : f32x4{};
  if (col == 0) p.out_lse[(int64_t)b * p.out_req_rows + head] = wsum > 0.f ? (mx + fast_log2(wsum)) * kLn2 : -INFINITY;
}

template <int DV, int PL, int DS = 1, int QPT = 1>
static hipError_t launch_split(const SplitReduceParams& p, hipStream_t stream) {
  using C = SplitCfg<DV, PL, DS, QPT>;
  dim3 grid(p.batch, (p.num_heads + C::kHpb - 1) / C::kHpb, DS);
  hipLaunchKernelGGL((split_reduce_kernel<DV, PL, DS, QPT>), grid, dim3(C::kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_split_reduce(const SplitReduceParams& p, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  // Expected pieces per request: about partitions / batch + 1.
  const int64_t per = (int64_t)p.num_parts / p.batch + 1;
  // Many requests: two quads per thread halve the waves of the grid (measured 25.6 ->
  // 19.1 us at B = 512; at B = 128 one quad per thread is faster, 16.8 against 21.7 us).
  const bool big = p.batch >= 256;
  if (p.v_dim == 512) {
    if (per <= 4) return big ? launch_split<512, 1, 1, 2>(p, stream) : launch_split<512, 1>(p, stream);
    if (per <= 16) return launch_split<512, 2>(p, stream);
    return launch_split<512, 8, 4>(p, stream);
  }
  if (per <= 4) return big ? launch_split<128, 1, 1, 2>(p, stream) : launch_split<128, 1>(p, stream);
  if (per <= 16) return launch_split<128, 4>(p, stream);
  return launch_split<128, 16>(p, stream);
}

// ------------------------------------------------------------------ N-way merge
// One thread per 4 consecutive output floats of one (request, head) row; the row's
// N LSE values are read by each of its threads (they stay in L1/L2).  kStream: the
// stacked partials are larger than the 256 MB last-level cache, so they are read in
// chunks of 8 ranks with every load issued before any is used and with the streaming
// (non-temporal) policy (measured at B = 512: 152 -> 99 us; for partials that the
// cache still holds, as at B = 128, the plain loop is faster: 27.5 against 29.8 us).
template <bool kStream>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_parts,
                                                    const float* __restrict__ lse_parts,
                                                    int32_t num_parts, int64_t rows, int32_t v_dim,
                                                    float* __restrict__ out_o,
                                                    float* __restrict__ out_lse) {
  const int quads = v_dim >> 2;
  const int64_t total = rows * quads;
  const int64_t part_stride = rows * v_dim;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = e / quads;
    const int qd = (int)(e - row * quads);
    const float* src = o_parts + row * v_dim + 4 * qd;
    float mx = -INFINITY;
    for (int r = 0; r < num_parts; ++r) mx = fmaxf(mx, lse_parts[(int64_t)r * rows + row]);
    f32x4 acc = f32x4{};
    float wsum = 0.f;
    if (mx != -INFINITY) {
      if constexpr (kStream) {
        for (int r0 = 0; r0 < num_parts; r0 += 8) {
          float l[8];
          f32x4 v[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int r = r0 + k;
            const bool ok = r < num_parts;
            l[k] = ok ? lse_parts[(int64_t)r * rows + row] : -INFINITY;
            v[k] = ok ? __builtin_nontemporal_load((const f32x4*)(src + r * part_stride)) : f32x4{};
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float wt = fast_exp2((l[k] - mx) * kLog2e);  // -inf -> 0
            wsum += wt;
            if (wt != 0.f) acc += wt * v[k];
          }
        }
      } else {
        for (int r = 0; r < num_parts; ++r) {
          const float l = lse_parts[(int64_t)r * rows + row];
          const float wt = fast_exp2((l - mx) * kLog2e);  // -inf -> 0
          wsum += wt;
          const f32x4 v = *(const f32x4*)(src + r * part_stride);
          if (wt != 0.f) acc += wt * v;
        }
      }
      acc *= 1.0f / wsum;
    }
    *(f32x4*)(out_o + row * v_dim + 4 * qd) = acc;
    if (qd == 0 && out_lse) out_lse[row] = mx == -INFINITY ? -INFINITY : mx + fast_log2(wsum) * kLn2;
  }
}

hipError_t launch_merge(const float* o_parts, const float* lse_parts, int32_t num_parts, int64_t rows,
                        int32_t v_dim, float* out_o, float* out_lse, hipStream_t stream) {
  const int64_t total = rows * (v_dim / 4);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 1 << 20) blocks = 1 << 20;
  const bool stream_parts = (int64_t)num_parts * rows * v_dim * 4 > ((int64_t)256 << 20);
  if (stream_parts)
    hipLaunchKernelGGL(merge_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, o_parts, lse_parts,
                       num_parts, rows, v_dim, out_o, out_lse);
  else
    hipLaunchKernelGGL(merge_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, o_parts, lse_parts,
                       num_parts, rows, v_dim, out_o, out_lse);
  return hipGetLastError();
}

// ------------------------------------------------------------------ workspace fill
// Zeroes `bytes` bytes (16 per thread, the tail byte-wise); a kernel rather than a
// memset so that the call can sit in a captured graph.
__global__ __launch_bounds__(256) void zero_fill_kernel(uint8_t* __restrict__ p, size_t bytes) {
  const size_t quads = bytes / 16;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < quads; i += (size_t)gridDim.x * blockDim.x)
    ((u32x4*)p)[i] = u32x4{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0 && threadIdx.x < bytes - quads * 16) p[quads * 16 + threadIdx.x] = 0;
}

hipError_t launch_zero_fill(void* ptr, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  size_t blocks = (bytes / 16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint8_t*)ptr, bytes);
  return hipGetLastError();
}

// ------------------------------------------------------------------ shard map kernels
__global__ void shard_map_kernel(const int32_t* __restrict__ seq_lens, int32_t batch, int32_t N,
                                 int32_t I, int32_t rank, int32_t* __restrict__ local_lens) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int32_t L = seq_lens[b];
  local_lens[b] = (int32_t)dcp_local_len(L < 0 ? 0 : L, N, I, rank);
}

hipError_t launch_shard_map(const int32_t* seq_lens, int32_t batch, int32_t N, int32_t I,
                            int32_t rank, int32_t* local_lens, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(shard_map_kernel, dim3((batch + 255) / 256), dim3(256), 0, stream, seq_lens,
                     batch, N, I, rank, local_lens);
  return hipGetLastError();
}

// Local page k of rank r = global page ((k / P) * N + r) * P + k % P, P = I / block_size.
__global__ void local_block_table_kernel(const int32_t* __restrict__ gbt, int32_t batch,
                                         int32_t max_global, int32_t N, int32_t P, int32_t rank,
                                         int32_t* __restrict__ lbt, int32_t max_local) {
  const int64_t total = (int64_t)batch * max_local;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = e / max_local;
    const int64_t k = e - b * max_local;
    const int64_t gk = ((k / P) * N + rank) * P + k % P;
    lbt[e] = gk < max_global ? gbt[b * max_global + gk] : -1;
  }
}

hipError_t launch_local_block_table(const int32_t* gbt, int32_t batch, int32_t max_global, int32_t N,
                                    int32_t P, int32_t rank, int32_t* lbt, int32_t max_local,
                                    hipStream_t stream) {
  const int64_t total = (int64_t)batch * max_local;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(local_block_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, gbt, batch,
                     max_global, N, P, rank, lbt, max_local);
  return hipGetLastError();
}

}  // namespace dcp
