// DCP-aware append of each request's newly decoded token to the KV cache.
//
// Every rank stores the KV of its own token positions only (vLLM blog "Efficient
// Decode Context Parallelism with vLLM for Long Context Workloads", Sec. 4 and
// Sec. 2.2), so the row of the token decoded last goes to the rank that owns its
// position, at the slot its local index names: position t = L - 1 of a request of
// new length L belongs to rank (t / I) % N at local index (t / (N I)) I + t % I.
#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {

struct AppendParams {
  const uint4* new_k;       // [B, row_k / 16] 16-byte chunks
  const uint4* new_v;       // [B, row_v / 16] (GQA) or null
  uint8_t* k_cache;
  uint8_t* v_cache;
  int64_t num_cache_blocks;
  const int32_t* block_table;
  int32_t max_blocks_per_seq;
  const int32_t* seq_lens;
  int32_t batch, rank, num_ranks, interleave, block_size;
  int32_t chunks_k, chunks_v;  // 16-byte chunks of one token's K row / V row
};

// One block per request; each thread copies 16-byte chunks of the new row.
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int b = blockIdx.x;
  const int64_t L = p.seq_lens[b];
  if (L <= 0) return;
  const int64_t t = L - 1;
  if (dcp_owner(t, p.num_ranks, p.interleave) != p.rank) return;
  const int64_t j = dcp_local_index(t, p.num_ranks, p.interleave);
  const int64_t k = j / p.block_size;
  if (k >= p.max_blocks_per_seq) return;
  const int32_t page = p.block_table[(int64_t)b * p.max_blocks_per_seq + k];
  if (page < 0 || (int64_t)page >= p.num_cache_blocks) return;
  const int64_t slot = (int64_t)page * p.block_size + (j - k * p.block_size);
  uint4* dk = (uint4*)p.k_cache + slot * p.chunks_k;
  const uint4* sk = p.new_k + (int64_t)b * p.chunks_k;
  for (int c = threadIdx.x; c < p.chunks_k; c += blockDim.x) dk[c] = sk[c];
  if (p.new_v) {
    uint4* dv = (uint4*)p.v_cache + slot * p.chunks_v;
    const uint4* sv = p.new_v + (int64_t)b * p.chunks_v;
    for (int c = threadIdx.x; c < p.chunks_v; c += blockDim.x) dv[c] = sv[c];
  }
}

hipError_t launch_append(const void* new_k, const void* new_v, void* k_cache, void* v_cache,
                         int64_t num_cache_blocks, const int32_t* block_table,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                         int32_t rank, int32_t num_ranks, int32_t interleave, int32_t block_size,
                         int32_t row_k_bytes, int32_t row_v_bytes, hipStream_t stream) {
  AppendParams p{};
  p.new_k = (const uint4*)new_k;
  p.new_v = (const uint4*)new_v;
  p.k_cache = (uint8_t*)k_cache;
  p.v_cache = (uint8_t*)v_cache;
  p.num_cache_blocks = num_cache_blocks;
  p.block_table = block_table;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.seq_lens = seq_lens;
  p.batch = batch;
  p.rank = rank;
  p.num_ranks = num_ranks;
  p.interleave = interleave;
  p.block_size = block_size;
  p.chunks_k = row_k_bytes / 16;
  p.chunks_v = row_v_bytes / 16;
  hipLaunchKernelGGL(append_kernel, dim3(batch), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dcp
