// Internal launch interface between the C ABI (dcp_api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcp_params.h"

namespace dcp {

constexpr int kMlaTile = 32;
constexpr int kGqaTile = 16;

int mla_heads_per_group(int num_q_heads);
int gqa_kv_heads_per_group(int num_kv_heads);

hipError_t launch_mla_partial(const PartialParams& p, hipStream_t stream);
hipError_t launch_gqa_partial(const PartialParams& p, hipStream_t stream);
hipError_t launch_split_reduce(const SplitReduceParams& p, hipStream_t stream);
hipError_t launch_merge_lse(const float* lse_parts, int32_t n, int64_t rows, float* out, hipStream_t s);
hipError_t launch_rescale(const float* o, const float* lse_r, const float* lse, int64_t rows,
                          int32_t v_dim, bool bf16, void* out, hipStream_t s);
hipError_t launch_sum_slice(const void* parts, bool bf16, int32_t n, int64_t batch, int32_t heads,
                            int32_t rank, int32_t v_dim, float* out, hipStream_t s);
hipError_t launch_append(const void* new_k, const void* new_v, void* k_cache, void* v_cache,
                         int64_t num_cache_blocks, const int32_t* block_table,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                         int32_t rank, int32_t num_ranks, int32_t interleave, int32_t block_size,
                         int32_t row_k_bytes, int32_t row_v_bytes, hipStream_t stream);
hipError_t launch_merge(const float* o_parts, const float* lse_parts, int32_t num_parts, int64_t rows,
                        int32_t v_dim, float* out_o, float* out_lse, hipStream_t stream);
hipError_t launch_shard_map(const int32_t* seq_lens, int32_t batch, int32_t N, int32_t I,
                            int32_t rank, int32_t* local_lens, hipStream_t stream);
hipError_t launch_zero_fill(void* ptr, size_t bytes, hipStream_t stream);
hipError_t launch_local_block_table(const int32_t* gbt, int32_t batch, int32_t max_global, int32_t N,
                                    int32_t P, int32_t rank, int32_t* lbt, int32_t max_local,
                                    hipStream_t stream);

}  // namespace dcp
