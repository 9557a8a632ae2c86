// C ABI of libdcp (declared in include/dcp.h): argument validation, work
// planning and kernel launches.  Host code only; the kernels live in the other
// .hip files of this directory.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "../../include/dcp.h"
#include "dcp_internal.h"
#include "dcp_params.h"
#include "dcp_shard.h"

namespace {

constexpr int32_t kMaxBatch = 1 << 16;
constexpr int32_t kMaxParts = 1 << 16;
constexpr int32_t kMaxMlaRows = 512;  // MLA score rows (query tokens x heads) per request
constexpr int64_t kMaxMtpRows = kMaxMlaRows;
constexpr int32_t kMaxGqaQueryTokens = 64;  // query tokens per request of a GQA multi-token call
constexpr int32_t kGqaMaxQueryBlock = 4;    // query tokens per GQA pass (MFMA column blocks)
constexpr int32_t kMaxDevices = 64;

// Cache of the compute-unit count per device (filled on first use; concurrent callers
// may both fill an entry, with the same value).
std::atomic<int> g_cu_count[kMaxDevices];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Shape checks shared by workspace sizing and the partial call.  Fills the
// number of head groups (work-groups per span) on success.
dcp_status_t check_desc(const dcp_attn_desc_t* d, int32_t* head_groups) {
  if (!d) return DCP_ERROR_INVALID_VALUE;
  if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->block_size < 1 || d->qk_dim < 1 ||
      d->v_dim < 1 || !(d->softmax_scale == d->softmax_scale) || isinf(d->softmax_scale))
    return DCP_ERROR_INVALID_VALUE;
  if (d->num_q_heads % d->num_kv_heads) return DCP_ERROR_INVALID_VALUE;
  if (d->kind == DCP_KV_MLA_LATENT) {
    if (d->num_kv_heads != 1) return DCP_ERROR_INVALID_VALUE;
    if (d->qk_dim != 576 || d->v_dim != 512) return DCP_ERROR_NOT_SUPPORTED;
    if (d->num_q_heads > kMaxMlaRows || d->block_size % dcp::kMlaTile) return DCP_ERROR_NOT_SUPPORTED;
    const int hpg = dcp::mla_heads_per_group(d->num_q_heads);
    *head_groups = (d->num_q_heads + hpg - 1) / hpg;
    return DCP_SUCCESS;
  }
  if (d->kind == DCP_KV_GQA) {
    if (d->qk_dim != 128 || d->v_dim != 128) return DCP_ERROR_NOT_SUPPORTED;
    if (d->num_q_heads / d->num_kv_heads > 16 || d->block_size % 16) return DCP_ERROR_NOT_SUPPORTED;
    *head_groups = d->num_kv_heads / dcp::gqa_kv_heads_per_group(d->num_kv_heads);
    return DCP_SUCCESS;
  }
  return DCP_ERROR_INVALID_VALUE;
}

}  // namespace

namespace dcp {
// Head-group policies (host side; the kernels' launchers use them too).
int mla_heads_per_group(int num_q_heads) { return num_q_heads <= 32 ? 32 : 64; }
int gqa_kv_heads_per_group(int num_kv_heads) {
  return num_kv_heads % 4 == 0 ? 4 : (num_kv_heads % 2 == 0 ? 2 : 1);
}
}  // namespace dcp

namespace {

// Tiles of work charged to each request a work-group touches (see the partition
// helpers in dcp_device.h): the query slice it reads and the fp32 output row it
// writes, in units of the tile bytes it streams.  MLA: a 64-head group moves 72 KiB
// of q and 128 KiB of O against 36 KiB per tile (about 5.6; 5 measured), a 32-head
// group half of that; GQA: 12 KiB per KV head against its 8 KiB of a 16-token tile.
int32_t request_weight(const dcp_attn_desc_t* d) {
  if (d->kind == DCP_KV_MLA_LATENT) return dcp::mla_heads_per_group(d->num_q_heads) == 64 ? 5 : 3;
  return 2;
}

int32_t default_parts(int32_t head_groups) {
  int cus = device_cu_count();
  if (cus <= 0) cus = 256;
  int32_t p = cus / head_groups;
  if (head_groups > 1) p = (p / 8) * 8;  // keeps the XCD-aware block mapping
  return p < 1 ? 1 : p;
}

// Workspace of a partial call: a 256-byte header (the device error word at offset 0, which
// dcp_workspace_init zeroes), the partition prefix, and the split pieces' LSEs and outputs.
struct WsLayout {
  size_t prefix, lse, o, total;
};

WsLayout ws_layout(int32_t batch, int32_t parts, int32_t heads, int32_t v_dim) {
  WsLayout l;
  l.prefix = 256;
  l.lse = l.prefix + align256(sizeof(int64_t) * (3 * (size_t)batch + 2));
  l.o = l.lse + align256(sizeof(float) * 2 * (size_t)parts * heads);
  l.total = l.o + align256(sizeof(float) * 2 * (size_t)parts * heads * v_dim);
  return l;
}

// Multi-token decode queries.  MLA: q_len query tokens of num_q_heads heads become
// q_len * num_q_heads score rows of one pass.  GQA: passes of up to four query tokens
// (the kernel keeps a KV head's query heads on the 16 MFMA columns, one column block
// per query token), so the head shapes are those of a single-token call and the
// workspace holds the pieces of one pass.
dcp_status_t check_q_len(const dcp_attn_desc_t* d, int32_t q_len, dcp_attn_desc_t* rows) {
  *rows = *d;
  if (q_len < 1) return DCP_ERROR_INVALID_VALUE;
  if (q_len == 1) return DCP_SUCCESS;
  if (d->kind == DCP_KV_GQA) return q_len <= kMaxGqaQueryTokens ? DCP_SUCCESS : DCP_ERROR_NOT_SUPPORTED;
  if (d->kind != DCP_KV_MLA_LATENT) return DCP_ERROR_INVALID_VALUE;
  if (d->num_q_heads < 1 || (int64_t)q_len * d->num_q_heads > kMaxMtpRows) return DCP_ERROR_NOT_SUPPORTED;
  rows->num_q_heads = q_len * d->num_q_heads;
  return DCP_SUCCESS;
}

// Piece rows per request in the workspace: the score rows of the pass with the most.
int32_t workspace_rows(const dcp_attn_desc_t* rows, int32_t q_len) {
  if (rows->kind != DCP_KV_GQA) return rows->num_q_heads;
  return (q_len < kGqaMaxQueryBlock ? q_len : kGqaMaxQueryBlock) * rows->num_q_heads;
}

dcp_status_t check_shard_args(int32_t num_ranks, int32_t interleave, int32_t rank) {
  if (num_ranks < 1 || interleave < 1 || rank < 0 || rank >= num_ranks) return DCP_ERROR_INVALID_VALUE;
  return DCP_SUCCESS;
}

dcp_status_t hip_status(hipError_t e) { return e == hipSuccess ? DCP_SUCCESS : DCP_ERROR_HIP; }

}  // namespace

extern "C" {

const char* dcp_status_string(dcp_status_t status) {
  switch (status) {
    case DCP_SUCCESS: return "DCP_SUCCESS";
    case DCP_ERROR_INVALID_VALUE: return "DCP_ERROR_INVALID_VALUE";
    case DCP_ERROR_NOT_SUPPORTED: return "DCP_ERROR_NOT_SUPPORTED";
    case DCP_ERROR_WORKSPACE: return "DCP_ERROR_WORKSPACE";
    case DCP_ERROR_HIP: return "DCP_ERROR_HIP";
    default: return "DCP_ERROR_UNKNOWN";
  }
}

dcp_status_t dcp_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes == 0 || ((uintptr_t)workspace & 255)) return DCP_ERROR_INVALID_VALUE;
  return hip_status(dcp::launch_zero_fill(workspace, workspace_bytes, (hipStream_t)stream));
}

dcp_status_t dcp_workspace_errors(const void* workspace, size_t workspace_bytes, uint32_t* error_bits,
                                  int32_t clear, void* stream) {
  if (!workspace || !error_bits || workspace_bytes < 256) return DCP_ERROR_INVALID_VALUE;
  hipStream_t s = (hipStream_t)stream;
  uint32_t word = 0;
  if (hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess)
    return DCP_ERROR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return DCP_ERROR_HIP;
  *error_bits = word;
  if (clear) {
    if (dcp::launch_zero_fill((void*)workspace, sizeof(uint32_t), s) != hipSuccess) return DCP_ERROR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return DCP_ERROR_HIP;
  }
  return DCP_SUCCESS;
}

dcp_status_t dcp_shard_map(const int32_t* seq_lens, int32_t batch, int32_t num_ranks,
                           int32_t interleave, int32_t rank, int32_t* local_lens,
                           int64_t* total_local, int32_t* max_local) {
  dcp_status_t st = check_shard_args(num_ranks, interleave, rank);
  if (st != DCP_SUCCESS) return st;
  if (batch < 0 || (batch > 0 && (!seq_lens || !local_lens))) return DCP_ERROR_INVALID_VALUE;
  for (int32_t b = 0; b < batch; ++b)
    if (seq_lens[b] < 0) return DCP_ERROR_INVALID_VALUE;
  int64_t total = 0;
  int32_t mx = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t lr = (int32_t)dcp_local_len(seq_lens[b], num_ranks, interleave, rank);
    local_lens[b] = lr;
    total += lr;
    mx = lr > mx ? lr : mx;
  }
  if (total_local) *total_local = total;
  if (max_local) *max_local = mx;
  return DCP_SUCCESS;
}

dcp_status_t dcp_shard_locate(const int64_t* positions, int64_t count, int32_t num_ranks,
                              int32_t interleave, int32_t* owner, int64_t* local_index) {
  if (num_ranks < 1 || interleave < 1 || count < 0) return DCP_ERROR_INVALID_VALUE;
  if (count > 0 && (!positions || !owner || !local_index)) return DCP_ERROR_INVALID_VALUE;
  for (int64_t i = 0; i < count; ++i)
    if (positions[i] < 0) return DCP_ERROR_INVALID_VALUE;
  for (int64_t i = 0; i < count; ++i) {
    owner[i] = dcp_owner(positions[i], num_ranks, interleave);
    local_index[i] = dcp_local_index(positions[i], num_ranks, interleave);
  }
  return DCP_SUCCESS;
}

dcp_status_t dcp_shard_global(const int64_t* local_index, int64_t count, int32_t num_ranks,
                              int32_t interleave, int32_t rank, int64_t* positions) {
  dcp_status_t st = check_shard_args(num_ranks, interleave, rank);
  if (st != DCP_SUCCESS) return st;
  if (count < 0 || (count > 0 && (!local_index || !positions))) return DCP_ERROR_INVALID_VALUE;
  for (int64_t i = 0; i < count; ++i)
    if (local_index[i] < 0) return DCP_ERROR_INVALID_VALUE;
  for (int64_t i = 0; i < count; ++i)
    positions[i] = dcp_global_index(local_index[i], num_ranks, interleave, rank);
  return DCP_SUCCESS;
}

dcp_status_t dcp_shard_map_device(const int32_t* seq_lens, int32_t batch, int32_t num_ranks,
                                  int32_t interleave, int32_t rank, int32_t* local_lens,
                                  void* stream) {
  dcp_status_t st = check_shard_args(num_ranks, interleave, rank);
  if (st != DCP_SUCCESS) return st;
  if (batch < 0 || (batch > 0 && (!seq_lens || !local_lens))) return DCP_ERROR_INVALID_VALUE;
  return hip_status(dcp::launch_shard_map(seq_lens, batch, num_ranks, interleave, rank, local_lens,
                                          (hipStream_t)stream));
}

dcp_status_t dcp_local_block_table(const int32_t* global_block_table, int32_t batch,
                                   int32_t max_global_blocks, int32_t num_ranks,
                                   int32_t interleave, int32_t block_size, int32_t rank,
                                   int32_t* local_block_table, int32_t max_local_blocks,
                                   void* stream) {
  dcp_status_t st = check_shard_args(num_ranks, interleave, rank);
  if (st != DCP_SUCCESS) return st;
  if (batch < 0 || max_global_blocks < 0 || max_local_blocks < 0 || block_size < 1)
    return DCP_ERROR_INVALID_VALUE;
  if ((int64_t)batch * max_local_blocks > 0 && (!local_block_table || (max_global_blocks > 0 && !global_block_table)))
    return DCP_ERROR_INVALID_VALUE;
  if (interleave % block_size) return DCP_ERROR_NOT_SUPPORTED;
  return hip_status(dcp::launch_local_block_table(global_block_table, batch, max_global_blocks,
                                                  num_ranks, interleave / block_size, rank,
                                                  local_block_table, max_local_blocks,
                                                  (hipStream_t)stream));
}

size_t dcp_decode_workspace_size_mtp(const dcp_attn_desc_t* desc, int32_t q_len, int32_t batch,
                                     int32_t num_partitions) {
  dcp_attn_desc_t d;
  if (!desc || check_q_len(desc, q_len, &d) != DCP_SUCCESS) return 0;
  int32_t groups = 0;
  if (check_desc(&d, &groups) != DCP_SUCCESS) return 0;
  if (batch < 0 || batch > kMaxBatch || num_partitions < 0 || num_partitions > kMaxParts) return 0;
  const int32_t parts = num_partitions ? num_partitions : default_parts(groups);
  return ws_layout(batch, parts, workspace_rows(&d, q_len), d.v_dim).total;
}

size_t dcp_decode_workspace_size(const dcp_attn_desc_t* desc, int32_t batch, int32_t num_partitions) {
  return dcp_decode_workspace_size_mtp(desc, 1, batch, num_partitions);
}

dcp_status_t dcp_decode_partial_mtp(const dcp_attn_desc_t* desc, int32_t q_len, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    int64_t num_cache_blocks, const int32_t* block_table,
                                    int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                    int32_t batch, int32_t rank, int32_t num_ranks,
                                    int32_t interleave, int32_t num_partitions, void* workspace,
                                    size_t workspace_bytes, float* out_o, float* out_lse,
                                    void* stream) {
  if (!desc) return DCP_ERROR_INVALID_VALUE;
  dcp_attn_desc_t d;  // one score row per (query token, head)
  dcp_status_t st = check_q_len(desc, q_len, &d);
  if (st != DCP_SUCCESS) return st;
  int32_t groups = 0;
  st = check_desc(&d, &groups);
  if (st != DCP_SUCCESS) return st;
  st = check_shard_args(num_ranks, interleave, rank);
  if (st != DCP_SUCCESS) return st;
  if (batch < 0 || batch > kMaxBatch || num_partitions < 0 || num_partitions > kMaxParts ||
      max_blocks_per_seq < 0 || num_cache_blocks < 0)
    return DCP_ERROR_INVALID_VALUE;
  if (batch == 0) return DCP_SUCCESS;
  if (!q || !k_cache || !block_table || !seq_lens || !out_o || !out_lse) return DCP_ERROR_INVALID_VALUE;
  if (num_cache_blocks < 1 || max_blocks_per_seq < 1) return DCP_ERROR_INVALID_VALUE;
  if ((d.kind == DCP_KV_MLA_LATENT) != (v_cache == nullptr)) return DCP_ERROR_INVALID_VALUE;
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15) return DCP_ERROR_INVALID_VALUE;
  if (((uintptr_t)out_o & 15) || ((uintptr_t)out_lse & 3)) return DCP_ERROR_INVALID_VALUE;
  const int32_t parts = num_partitions ? num_partitions : default_parts(groups);
  const WsLayout wl = ws_layout(batch, parts, workspace_rows(&d, q_len), d.v_dim);
  if (!workspace || ((uintptr_t)workspace & 255) || workspace_bytes < wl.total) return DCP_ERROR_WORKSPACE;

  uint8_t* ws = (uint8_t*)workspace;
  dcp::PartialParams p{};
  p.q = (const uint16_t*)q;
  p.k_cache = (const uint8_t*)k_cache;
  p.v_cache = (const uint8_t*)v_cache;
  p.num_cache_blocks = num_cache_blocks;
  p.block_table = block_table;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.batch = batch;
  p.num_q_heads = d.num_q_heads;
  p.num_kv_heads = d.num_kv_heads;
  p.block_size = d.block_size;
  p.num_head_groups = groups;
  p.q_len = q_len;
  p.heads_per_token = desc->num_q_heads;
  p.q_block = 1;
  p.scale_log2 = d.softmax_scale * 1.4426950408889634f;
  p.part.seq_lens = seq_lens;
  p.part.batch = batch;
  p.part.rank = rank;
  p.part.num_ranks = num_ranks;
  p.part.interleave = interleave;
  p.part.max_blocks_per_seq = max_blocks_per_seq;
  p.part.block_size = d.block_size;
  p.part.tile = d.kind == DCP_KV_MLA_LATENT ? dcp::kMlaTile : dcp::kGqaTile;
  p.part.num_parts = parts;
  p.part.req_weight = request_weight(&d);
  p.part.len_offset = 0;
  // span w runs on XCD w % 8 with one head group (see block_to_span)
  p.part.xcd_weighted = (groups == 1 && parts % 8 == 0) ? 1 : 0;
  p.out_o = out_o;
  p.out_lse = out_lse;
  p.q_req_stride = (int64_t)d.num_q_heads * d.qk_dim;
  p.out_req_rows = d.num_q_heads;
  p.ws_err = (uint32_t*)ws;
  p.ws_prefix = (int64_t*)(ws + wl.prefix);
  p.ws_lse = (float*)(ws + wl.lse);
  p.ws_o = (float*)(ws + wl.o);

  dcp::SplitReduceParams r{};
  r.ws_prefix = p.ws_prefix;
  r.ws_lse = p.ws_lse;
  r.ws_o = p.ws_o;
  r.batch = batch;
  r.num_heads = d.num_q_heads;
  r.v_dim = d.v_dim;
  r.num_parts = parts;
  r.req_weight = p.part.req_weight;
  r.out_req_rows = d.num_q_heads;
  r.xcd_weighted = p.part.xcd_weighted;
  r.out_o = out_o;
  r.out_lse = out_lse;

  hipStream_t s = (hipStream_t)stream;
  if (d.kind == DCP_KV_MLA_LATENT) {
    if (dcp::launch_mla_partial(p, s) != hipSuccess) return DCP_ERROR_HIP;
    return hip_status(dcp::launch_split_reduce(r, s));
  }
  // GQA: query token i of a request at global length L sees the positions <= L - q_len
  // + i.  Passes of qb = 4, 2 or 1 consecutive query tokens i0 .. i0 + qb - 1: the
  // partition covers the pass's newest token's positions (length L - (q_len - i0 - qb))
  // and the kernel masks, for each older token, the newest positions it may not see.
  // Each pass has its own slices of q [B, q_len, H, D] and of the outputs
  // [B, q_len, H, .]; the passes reuse the workspace in stream order.
  p.q_len = 1;
  p.q_req_stride = (int64_t)q_len * d.num_q_heads * d.qk_dim;
  p.out_req_rows = (int64_t)q_len * d.num_q_heads;
  r.out_req_rows = p.out_req_rows;
  for (int32_t i0 = 0; i0 < q_len;) {
    const int32_t left = q_len - i0;
    const int32_t qb = left >= 4 ? 4 : (left >= 2 ? 2 : 1);
    p.q_block = qb;
    p.part.len_offset = q_len - i0 - qb;
    // a request's query slices and output rows grow with the pass's query tokens
    p.part.req_weight = request_weight(&d) * qb;
    r.req_weight = p.part.req_weight;
    p.q = (const uint16_t*)q + (int64_t)i0 * d.num_q_heads * d.qk_dim;
    p.out_o = out_o + (int64_t)i0 * d.num_q_heads * d.v_dim;
    p.out_lse = out_lse + (int64_t)i0 * d.num_q_heads;
    r.num_heads = qb * d.num_q_heads;
    r.out_o = p.out_o;
    r.out_lse = p.out_lse;
    if (dcp::launch_gqa_partial(p, s) != hipSuccess) return DCP_ERROR_HIP;
    if (dcp::launch_split_reduce(r, s) != hipSuccess) return DCP_ERROR_HIP;
    i0 += qb;
  }
  return DCP_SUCCESS;
}

dcp_status_t dcp_decode_partial(const dcp_attn_desc_t* desc, const void* q, const void* k_cache,
                                const void* v_cache, int64_t num_cache_blocks,
                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, int32_t batch, int32_t rank,
                                int32_t num_ranks, int32_t interleave, int32_t num_partitions,
                                void* workspace, size_t workspace_bytes, float* out_o,
                                float* out_lse, void* stream) {
  return dcp_decode_partial_mtp(desc, 1, q, k_cache, v_cache, num_cache_blocks, block_table,
                                max_blocks_per_seq, seq_lens, batch, rank, num_ranks, interleave,
                                num_partitions, workspace, workspace_bytes, out_o, out_lse, stream);
}

dcp_status_t dcp_append_kv(const dcp_attn_desc_t* desc, const void* new_k, const void* new_v,
                           void* k_cache, void* v_cache, int64_t num_cache_blocks,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t batch, int32_t rank,
                           int32_t num_ranks, int32_t interleave, void* stream) {
  int32_t groups = 0;
  dcp_status_t st = check_desc(desc, &groups);
  if (st != DCP_SUCCESS) return st;
  st = check_shard_args(num_ranks, interleave, rank);
  if (st != DCP_SUCCESS) return st;
  if (batch < 0 || batch > kMaxBatch || max_blocks_per_seq < 1 || num_cache_blocks < 1)
    return DCP_ERROR_INVALID_VALUE;
  if (batch == 0) return DCP_SUCCESS;
  const bool mla = desc->kind == DCP_KV_MLA_LATENT;
  if (!new_k || !k_cache || !block_table || !seq_lens) return DCP_ERROR_INVALID_VALUE;
  if (mla != (new_v == nullptr) || mla != (v_cache == nullptr)) return DCP_ERROR_INVALID_VALUE;
  if (((uintptr_t)new_k | (uintptr_t)new_v | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15)
    return DCP_ERROR_INVALID_VALUE;
  const int32_t row_k = desc->num_kv_heads * desc->qk_dim * 2;
  const int32_t row_v = mla ? 0 : desc->num_kv_heads * desc->v_dim * 2;
  return hip_status(dcp::launch_append(new_k, new_v, k_cache, v_cache, num_cache_blocks, block_table,
                                       max_blocks_per_seq, seq_lens, batch, rank, num_ranks,
                                       interleave, desc->block_size, row_k, row_v,
                                       (hipStream_t)stream));
}

dcp_status_t dcp_merge(const float* o_parts, const float* lse_parts, int32_t num_parts,
                       int32_t batch, int32_t num_heads, int32_t v_dim, float* out_o,
                       float* out_lse, void* stream) {
  if (num_parts < 1 || batch < 0 || num_heads < 0 || v_dim < 4 || v_dim % 4) return DCP_ERROR_INVALID_VALUE;
  const int64_t rows = (int64_t)batch * num_heads;
  if (rows == 0) return DCP_SUCCESS;
  if (!o_parts || !lse_parts || !out_o) return DCP_ERROR_INVALID_VALUE;
  if (((uintptr_t)o_parts | (uintptr_t)out_o) & 15) return DCP_ERROR_INVALID_VALUE;
  return hip_status(dcp::launch_merge(o_parts, lse_parts, num_parts, rows, v_dim, out_o, out_lse,
                                      (hipStream_t)stream));
}

dcp_status_t dcp_merge_lse(const float* lse_parts, int32_t num_parts, int32_t batch,
                           int32_t num_heads, float* out_lse, void* stream) {
  if (num_parts < 1 || batch < 0 || num_heads < 0) return DCP_ERROR_INVALID_VALUE;
  const int64_t rows = (int64_t)batch * num_heads;
  if (rows == 0) return DCP_SUCCESS;
  if (!lse_parts || !out_lse) return DCP_ERROR_INVALID_VALUE;
  return hip_status(dcp::launch_merge_lse(lse_parts, num_parts, rows, out_lse, (hipStream_t)stream));
}

dcp_status_t dcp_rescale_partial(const float* o_r, const float* lse_r, const float* lse,
                                 int32_t batch, int32_t num_heads, int32_t v_dim,
                                 int32_t out_dtype, void* out, void* stream) {
  if (batch < 0 || num_heads < 0 || v_dim < 4 || v_dim % 4) return DCP_ERROR_INVALID_VALUE;
  if (out_dtype != DCP_DTYPE_F32 && out_dtype != DCP_DTYPE_BF16) return DCP_ERROR_INVALID_VALUE;
  const int64_t rows = (int64_t)batch * num_heads;
  if (rows == 0) return DCP_SUCCESS;
  if (!o_r || !lse_r || !lse || !out) return DCP_ERROR_INVALID_VALUE;
  if (((uintptr_t)o_r & 15) || ((uintptr_t)out & (out_dtype == DCP_DTYPE_F32 ? 15 : 7)))
    return DCP_ERROR_INVALID_VALUE;
  return hip_status(dcp::launch_rescale(o_r, lse_r, lse, rows, v_dim, out_dtype == DCP_DTYPE_BF16, out,
                                        (hipStream_t)stream));
}

dcp_status_t dcp_sum_head_slice(const void* scaled_parts, int32_t in_dtype, int32_t num_parts,
                                int32_t batch, int32_t num_heads, int32_t v_dim, int32_t rank,
                                float* out, void* stream) {
  if (num_parts < 1 || batch < 0 || num_heads < 0 || v_dim < 4 || v_dim % 4) return DCP_ERROR_INVALID_VALUE;
  if (num_heads % num_parts || rank < 0 || rank >= num_parts) return DCP_ERROR_INVALID_VALUE;
  if (in_dtype != DCP_DTYPE_F32 && in_dtype != DCP_DTYPE_BF16) return DCP_ERROR_INVALID_VALUE;
  if ((int64_t)batch * num_heads == 0) return DCP_SUCCESS;
  if (!scaled_parts || !out) return DCP_ERROR_INVALID_VALUE;
  if (((uintptr_t)scaled_parts & (in_dtype == DCP_DTYPE_F32 ? 15 : 7)) || ((uintptr_t)out & 15))
    return DCP_ERROR_INVALID_VALUE;
  return hip_status(dcp::launch_sum_slice(scaled_parts, in_dtype == DCP_DTYPE_BF16, num_parts, batch,
                                          num_heads, rank, v_dim, out, (hipStream_t)stream));
}

}  // extern "C"
