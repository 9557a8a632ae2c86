// Parameter blocks passed by value to the kernels (plain data, host and device).
#pragma once
#include <stdint.h>

namespace dcp {

// How a rank's tiles are cut into work partitions (see the partition helpers in
// dcp_device.h).
struct PartitionArgs {
  const int32_t* seq_lens;  // [B] global lengths (device)
  int32_t batch;
  int32_t rank, num_ranks, interleave;
  int32_t max_blocks_per_seq, block_size;
  int32_t tile;             // tokens per tile
  int32_t num_parts;        // P
  int32_t req_weight;       // tiles of work charged to each request with local tokens
  int32_t len_offset;       // subtracted from every seq_lens entry (a query token's causal length)
  int32_t xcd_weighted;     // spans weighted by the speed of the XCD they run on (see span_units)
};

struct PartialParams {
  const uint16_t* q;        // [B, H, qk_dim] bf16
  const uint8_t* k_cache;   // page pool (bytes)
  const uint8_t* v_cache;   // GQA V page pool (bytes); MLA: unused
  int64_t num_cache_blocks;
  const int32_t* block_table;
  int32_t max_blocks_per_seq;
  int32_t batch, num_q_heads, num_kv_heads, block_size;
  int32_t num_head_groups;  // work-groups sharing one span (disjoint head sets)
  int32_t q_len;            // query tokens per request (1: single-token decode)
  int32_t heads_per_token;  // query heads per query token; rows = q_len * heads_per_token
  int32_t q_block;          // GQA: query tokens of this pass (1, 2 or 4), on consecutive MFMA
                            // column blocks; its pieces have q_block * num_q_heads rows
  float scale_log2;         // softmax_scale * log2(e)
  PartitionArgs part;
  float* out_o;             // [B, H, v_dim]
  float* out_lse;           // [B, H]
  int64_t q_req_stride;     // GQA: query elements between consecutive requests (q_len * H * qk_dim;
                            // the pass's q_block tokens are consecutive, H * qk_dim apart)
  int64_t out_req_rows;     // GQA: output rows between consecutive requests (q_len * H)
  uint32_t* ws_err;         // device error word (dcp_device_error_t bits)
  int64_t* ws_prefix;       // [3 B + 2]: tile prefix, weighted prefix, span range of each request
  float* ws_lse;            // [2P, H]
  float* ws_o;              // [2P, H, v_dim]
};

struct SplitReduceParams {
  const int64_t* ws_prefix;  // [3 B + 2]: first tile of each request (total at [B]), its
                             // weighted position (weighted total at [2 B + 1]), then the
                             // spans of its first and last tiles (w_first << 32 | w_last)
  const float* ws_lse;       // [2P, H]
  const float* ws_o;         // [2P, H, v_dim]
  int32_t batch, num_heads, v_dim, num_parts, req_weight;
  int32_t xcd_weighted;      // as PartitionArgs::xcd_weighted of the partial call
  int64_t out_req_rows;      // output rows between consecutive requests (num_heads, or q_len *
                             // query heads for a pass of a multi-token GQA call)
  float* out_o;              // [B, H, v_dim]
  float* out_lse;            // [B, H]
};

}  // namespace dcp
