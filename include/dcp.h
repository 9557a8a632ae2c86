/*
 * dcp.h — C ABI of libdcp: single-token decode attention over one rank's
 * sequence-dimension shard of a paged KV cache, and the log-sum-exp merge that
 * turns the shards' partial results into the full-context result.
 *
 * The operation is Decode Context Parallelism as the vLLM blog "Efficient Decode
 * Context Parallelism with vLLM for Long Context Workloads" describes it:
 *   - Sec. 4 ("What is DCP?"): the KV cache of every request is split along the
 *     sequence dimension; each GPU holds and reads the cache of a subset of the
 *     token positions (Sec. 2.2: 1/N of every request's KV).
 *   - Sec. 4.1 ("Decode Context Parallelism Process"), "Compute": each GPU attends
 *     the full single-token query against its local KV slice and produces a
 *     partial output plus a log-sum-exp (LSE) per head; then the LSE values
 *     reweight and merge the partials (the rescaling online softmax also uses) into
 *     the exact full-context result.
 *   - Sec. 5.3 (MLA backend): one latent KV vector shared by every query head;
 *     Sec. 5.4 (GQA backend): each KV head is shared by a group of query heads.
 *   - The vLLM-Ascend "Decode Context Parallel Guide", Constraints: the KV cache
 *     interleave size (cp_kv_cache_interleave_size) and the page (block) size.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   Sharding.   Global token position t of a request belongs to rank
 *               (t / I) % N for interleave size I >= 1 and N >= 1 ranks.  A rank
 *               stores its tokens densely in ascending global order: local index
 *               j = (t / (N*I)) * I + t % I.  A request of global length L holds
 *               L_r = (L / (N*I)) * I + clamp(L % (N*I) - r*I, 0, I) tokens on rank r.
 *   Ownership.  The caller allocates every buffer.  The library allocates no
 *               memory, keeps no pointer after a call returns and has no mutable
 *               global state; calls are re-entrant.
 *   Memory.     "device" pointers are HIP device memory of the current device;
 *               "host" pointers are ordinary host memory.  Tensors are dense,
 *               row-major, with the shapes given.
 *   Streams.    `stream` is a hipStream_t (NULL = the default stream).  Device
 *               work is enqueued on it; no call synchronises the device.
 *   Errors.     Arguments the host can check are validated before anything is
 *               enqueued; on failure a status other than DCP_SUCCESS is returned
 *               and nothing runs.  DCP_ERROR_HIP reports a failed launch.
 *               Device-resident values the host cannot see (page ids, lengths)
 *               are clamped by the kernels so that no access leaves its buffer:
 *               a block-table entry outside [0, num_cache_blocks) is read as page
 *               0, a negative seq_lens entry as 0, and a rank never reads more than
 *               max_blocks_per_seq pages of a request.  Such inputs give
 *               meaningless numbers, never a fault; the partial-attention calls
 *               also record each such event as a bit of the workspace's device
 *               error word (dcp_workspace_errors below).
 */
#ifndef DCP_H_
#define DCP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DCP_SUCCESS = 0,
  DCP_ERROR_INVALID_VALUE = 1, /* a null pointer, a size or an index out of range */
  DCP_ERROR_NOT_SUPPORTED = 2, /* a valid shape the library has no kernel for */
  DCP_ERROR_WORKSPACE = 3,     /* workspace missing or smaller than required */
  DCP_ERROR_HIP = 4            /* the HIP runtime reported an error */
} dcp_status_t;

typedef enum {
  /* MLA (blog Sec. 5.3): one latent KV head; the cache row is the latent vector
   * (qk_dim = 576 = 512 latent + 64 rope); K is the whole row and V its first
   * v_dim (= 512) entries.  The query is in the same latent space. */
  DCP_KV_MLA_LATENT = 0,
  /* GQA (blog Sec. 5.4): num_kv_heads KV heads; query head h reads KV head
   * h / (num_q_heads / num_kv_heads).  K and V live in separate caches. */
  DCP_KV_GQA = 1
} dcp_kv_kind_t;

typedef struct {
  int32_t kind;          /* dcp_kv_kind_t */
  int32_t num_q_heads;   /* H */
  int32_t num_kv_heads;  /* 1 for MLA; H % num_kv_heads == 0 for GQA */
  int32_t qk_dim;        /* 576 for MLA, 128 for GQA */
  int32_t v_dim;         /* 512 for MLA, 128 for GQA */
  int32_t block_size;    /* tokens per KV page */
  float softmax_scale;   /* logits are softmax_scale * (q . k), applied in fp32 */
} dcp_attn_desc_t;

/* Human-readable name of a status code (static storage). */
const char* dcp_status_string(dcp_status_t status);

/* ------------------------------------------------------------------ shard map
 * Blog Sec. 4 and Sec. 2.2; interleave size from the vLLM-Ascend guide.     */

/* Local lengths of one rank (host).
 *   seq_lens   host int32 [batch]: global request lengths (including the
 *              current decode token); must be >= 0.
 *   local_lens host int32 [batch], written: L_r of every request.
 *   total_local, max_local: optional (NULL allowed) host outputs, the sum and
 *              the maximum of local_lens.
 * Errors: INVALID_VALUE if batch < 0, num_ranks < 1, interleave < 1,
 * rank not in [0, num_ranks), a needed pointer is NULL, or a length < 0.   */
dcp_status_t dcp_shard_map(const int32_t* seq_lens, int32_t batch, int32_t num_ranks,
                           int32_t interleave, int32_t rank, int32_t* local_lens,
                           int64_t* total_local, int32_t* max_local);

/* Owner rank and local index of global positions (host).
 *   positions host int64 [count] (>= 0); owner host int32 [count] and
 *   local_index host int64 [count] are written.                              */
dcp_status_t dcp_shard_locate(const int64_t* positions, int64_t count, int32_t num_ranks,
                              int32_t interleave, int32_t* owner, int64_t* local_index);

/* Global position of rank-local indices (host): the inverse of dcp_shard_locate.
 *   local_index host int64 [count] (>= 0); positions host int64 [count] written. */
dcp_status_t dcp_shard_global(const int64_t* local_index, int64_t count, int32_t num_ranks,
                              int32_t interleave, int32_t rank, int64_t* positions);

/* Local lengths of one rank computed on the device with the same code the
 * attention kernels use.  seq_lens, local_lens: device int32 [batch].         */
dcp_status_t dcp_shard_map_device(const int32_t* seq_lens, int32_t batch, int32_t num_ranks,
                                  int32_t interleave, int32_t rank, int32_t* local_lens,
                                  void* stream);

/* A rank's block table viewed out of a request-global block table (device),
 * for page-aligned interleaving: requires interleave % block_size == 0, so each
 * global page lies wholly on one rank.  With P = interleave / block_size, local
 * page k of rank r is global page ((k / P) * N + r) * P + k % P.
 *   global_block_table device int32 [batch, max_global_blocks]
 *   local_block_table  device int32 [batch, max_local_blocks], written; entries
 *                      whose global page falls outside the table are set to -1.
 * Errors: INVALID_VALUE for bad sizes/rank/pointers; NOT_SUPPORTED if
 * interleave % block_size != 0.                                               */
dcp_status_t dcp_local_block_table(const int32_t* global_block_table, int32_t batch,
                                   int32_t max_global_blocks, int32_t num_ranks,
                                   int32_t interleave, int32_t block_size, int32_t rank,
                                   int32_t* local_block_table, int32_t max_local_blocks,
                                   void* stream);

/* ------------------------------------------------------------------ partial attention
 * Blog Sec. 4.1 "Compute", Sec. 5.3 (MLA), Sec. 5.4 (GQA).                 */

/* Device error word of a workspace: bits the partial-attention kernels set when they
 * clamp a device-resident value (see "Errors" above).  The bits accumulate over calls
 * until cleared. */
typedef enum {
  DCP_DEVERR_PAGE_ID = 1u,     /* a block-table entry outside [0, num_cache_blocks) was read */
  DCP_DEVERR_TABLE_SHORT = 2u, /* a request's local length exceeded max_blocks_per_seq pages */
  DCP_DEVERR_NEG_LENGTH = 4u   /* a seq_lens entry was negative */
} dcp_device_error_t;

/* Zero a workspace for dcp_decode_partial / dcp_decode_partial_mtp (device; enqueued
 * on `stream`, no allocation), so that its device error word starts clear.
 * Errors: INVALID_VALUE for a NULL or misaligned workspace or zero bytes; HIP. */
dcp_status_t dcp_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Read the device error word of a workspace into *error_bits (host), after the work
 * enqueued on `stream` so far; clears the word if `clear` is nonzero.  Synchronises
 * `stream` (a diagnostic, not for the decode loop).
 * Errors: INVALID_VALUE for NULL pointers or a workspace smaller than 256 bytes; HIP. */
dcp_status_t dcp_workspace_errors(const void* workspace, size_t workspace_bytes, uint32_t* error_bits,
                                  int32_t clear, void* stream);

/* Workspace bytes dcp_decode_partial needs for `batch` requests split into
 * `num_partitions` token-balanced work partitions (0 = the library's default
 * for the current device).  Returns 0 for an invalid or unsupported desc.     */
size_t dcp_decode_workspace_size(const dcp_attn_desc_t* desc, int32_t batch,
                                 int32_t num_partitions);

/* One rank's partial decode attention.
 *   q            device bf16 [batch, H, qk_dim]: the full (gathered) query.
 *   k_cache      device bf16, this rank's page pool:
 *                  MLA: [num_cache_blocks, block_size, qk_dim] latent rows;
 *                  GQA: [num_cache_blocks, block_size, num_kv_heads, qk_dim].
 *   v_cache      MLA: must be NULL (V is the first v_dim entries of each latent
 *                row); GQA: device bf16 [num_cache_blocks, block_size,
 *                num_kv_heads, v_dim].
 *   block_table  device int32 [batch, max_blocks_per_seq]: entry k of request b
 *                is the pool page holding the rank's local tokens
 *                [k*block_size, (k+1)*block_size) of that request.
 *   seq_lens     device int32 [batch]: GLOBAL lengths; the kernel derives each
 *                request's local length from (seq_lens, rank, num_ranks,
 *                interleave).
 *   num_partitions  work partitions per head group (0 = default).  The rank's
 *                local tokens are cut into this many consecutive ranges of equal
 *                work across the batch (tiles of 32 tokens, each request also
 *                charged a few tiles for its query and output traffic); a
 *                request cut between partitions is reduced in a second kernel
 *                (split-K).
 *   workspace    device, >= dcp_decode_workspace_size(desc, batch, num_partitions)
 *                bytes, 256-byte aligned.  Its first 256 bytes hold the device error
 *                word, meaningful once dcp_workspace_init has zeroed it; nothing else
 *                in it needs initialisation.  Calls that share a workspace must be
 *                ordered (one stream); a workspace is not shared between calls that
 *                may run concurrently.
 *   out_o        device fp32 [batch, H, v_dim], written: normalised partial output
 *                O_r = sum_t p_t v_t / sum_t p_t over the rank's tokens.
 *   out_lse      device fp32 [batch, H], written: LSE_r = ln sum_t exp(s_t),
 *                s_t = softmax_scale * (q . k_t).
 *   A request with no local tokens gets O_r = 0 and LSE_r = -inf.
 * Arithmetic: scores, softmax statistics and accumulation in fp32; the softmax
 * weights enter the P.V product as bf16, plus their bf16 low part in the tiles
 * where a weight is a sizeable share of its row (requests of up to 256 local
 * tokens, dominant tokens), which keeps |dO| against exact attention near 1e-3
 * or below on bf16 inputs of unit scale.
 * Supported: MLA with qk_dim 576, v_dim 512, 1 <= H <= 512, block_size a
 * multiple of 32; GQA with qk_dim = v_dim = 128, H / num_kv_heads <= 16,
 * block_size a multiple of 16.
 * Errors: INVALID_VALUE, NOT_SUPPORTED, WORKSPACE, HIP (nothing runs on error). */
dcp_status_t dcp_decode_partial(const dcp_attn_desc_t* desc, const void* q, const void* k_cache,
                                const void* v_cache, int64_t num_cache_blocks,
                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, int32_t batch, int32_t rank,
                                int32_t num_ranks, int32_t interleave, int32_t num_partitions,
                                void* workspace, size_t workspace_bytes, float* out_o,
                                float* out_lse, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): dcp_decode_partial with the library's
 * own static device scratch (72 MiB per device, held until the process ends) in place of
 * the caller's workspace.  Arguments, outputs and errors as for dcp_decode_partial; a
 * call whose workspace (dcp_decode_workspace_size) would exceed the scratch returns
 * DCP_ERROR_WORKSPACE and runs nothing.  Allocates nothing: the first call on a device
 * zeroes that device's scratch on `stream`.  Every call on a device shares its scratch,
 * so calls that overlap on one GPU (different streams, or concurrent host threads
 * without stream order between their work) race and give wrong results.  The device
 * error word of the scratch (see dcp_workspace_errors) is not exposed: callers that
 * want the device-side checks pass their own workspace to dcp_decode_partial. */
dcp_status_t dcp_decode_partial_noalloc(const dcp_attn_desc_t* desc, const void* q, const void* k_cache,
                                        const void* v_cache, int64_t num_cache_blocks,
                                        const int32_t* block_table, int32_t max_blocks_per_seq,
                                        const int32_t* seq_lens, int32_t batch, int32_t rank,
                                        int32_t num_ranks, int32_t interleave, int32_t num_partitions,
                                        float* out_o, float* out_lse, void* stream);

/* Multi-token decode queries (speculative decoding / multi-token prediction; blog
 * Sec. 6): q_len >= 1 query tokens per request, the request's last q_len positions,
 * whose K/V rows are already in the cache (seq_lens counts them).  Query i (global
 * position L - q_len + i) attends the positions <= L - q_len + i, causally by GLOBAL
 * position, so on each rank it sees the local tokens up to that position; a query
 * that sees none of the rank's tokens gets O_r = 0, LSE_r = -inf, and dcp_merge over
 * the ranks gives causal attention over the whole context.  q_len = 1 is
 * dcp_decode_partial.
 *   q        device bf16 [batch, q_len, H, qk_dim]
 *   out_o    device fp32 [batch, q_len, H, v_dim], written
 *   out_lse  device fp32 [batch, q_len, H], written
 *   workspace  >= dcp_decode_workspace_size_mtp(desc, q_len, batch, num_partitions)
 * Every other argument as for dcp_decode_partial.
 * Supported: MLA with q_len * H <= 512, computed in one pass with the q_len * H
 * (query token, head) pairs as score rows; GQA with q_len <= 64, computed in passes
 * of four consecutive query tokens (then two, then one for what is left), each pass
 * reading the rank's pages of its newest token's causal length once for all its
 * tokens.
 * Errors: INVALID_VALUE (q_len < 1, and as dcp_decode_partial), NOT_SUPPORTED,
 * WORKSPACE (nothing runs on these), HIP (a GQA call that fails to launch pass i
 * leaves passes 0 .. i-1 enqueued).                                            */
size_t dcp_decode_workspace_size_mtp(const dcp_attn_desc_t* desc, int32_t q_len, int32_t batch,
                                     int32_t num_partitions);
dcp_status_t dcp_decode_partial_mtp(const dcp_attn_desc_t* desc, int32_t q_len, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    int64_t num_cache_blocks, const int32_t* block_table,
                                    int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                    int32_t batch, int32_t rank, int32_t num_ranks,
                                    int32_t interleave, int32_t num_partitions, void* workspace,
                                    size_t workspace_bytes, float* out_o, float* out_lse,
                                    void* stream);

/* ------------------------------------------------------------------ KV append
 * Blog Sec. 4 ("What is DCP?") and Sec. 2.2: every rank stores the KV of its own
 * token positions only, so the KV row of a newly decoded token goes to the one
 * rank that owns its position.  With seq_lens counting the new token, request b's
 * new token sits at global position t = seq_lens[b] - 1; its owner is
 * (t / I) % N, its local index j = (t / (N*I)) * I + t % I, and its row is
 * written to slot j % block_size of page block_table[b][j / block_size].
 *
 * Each rank calls this on its own cache with the same arguments apart from
 * `rank`, `block_table` and the caches; a call writes the rows of the requests the
 * rank owns and nothing else.
 *   new_k     device bf16 [batch, qk_dim] (MLA: the 576-dim latent row) or
 *             [batch, num_kv_heads, qk_dim] (GQA)
 *   new_v     GQA: device bf16 [batch, num_kv_heads, v_dim]; MLA: NULL
 *   k_cache, v_cache  the rank's page pools, laid out as for dcp_decode_partial
 *             (v_cache NULL for MLA); num_cache_blocks pages.
 *   block_table  device int32 [batch, max_blocks_per_seq], the rank's pages.
 *   seq_lens  device int32 [batch]: global lengths including the new token.
 * A request with seq_lens[b] <= 0, a local index past max_blocks_per_seq pages,
 * or a page id outside [0, num_cache_blocks) gets no write (nothing else is
 * touched).  The rows written must not be read by work running concurrently.
 * Supported: the shapes dcp_decode_partial supports.
 * Errors: INVALID_VALUE, NOT_SUPPORTED, HIP (nothing runs on error).          */
dcp_status_t dcp_append_kv(const dcp_attn_desc_t* desc, const void* new_k, const void* new_v,
                           void* k_cache, void* v_cache, int64_t num_cache_blocks,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t batch, int32_t rank,
                           int32_t num_ranks, int32_t interleave, void* stream);

/* ------------------------------------------------------------------ merge
 * Blog Sec. 4.1, "AllGather + ReduceScatter": the LSE values reweight and merge
 * the partials.  LSE = ln sum_r exp(LSE_r);  O = sum_r exp(LSE_r - LSE) O_r.
 * Parts with LSE_r = -inf carry no weight; if all are -inf, O = 0, LSE = -inf. */

/* N-way merge of num_parts partial results.
 *   o_parts   device fp32 [num_parts, batch, H, v_dim]
 *   lse_parts device fp32 [num_parts, batch, H]
 *   out_o     device fp32 [batch, H, v_dim], written (must not alias the inputs)
 *   out_lse   device fp32 [batch, H], written (nullable: LSE not stored).
 * Errors: INVALID_VALUE for num_parts < 1, negative sizes, v_dim not a
 * multiple of 4 or NULL inputs.                                              */
dcp_status_t dcp_merge(const float* o_parts, const float* lse_parts, int32_t num_parts,
                       int32_t batch, int32_t num_heads, int32_t v_dim, float* out_o,
                       float* out_lse, void* stream);

/* The same merge as the per-rank steps of a multi-GPU group (blog Sec. 4.1,
 * "AllGather + ReduceScatter"): (1) after an all-gather of the LSE_r every rank
 * computes the global LSE; (2) each rank scales its own partial by its share
 * exp(LSE_r - LSE); (3) a reduce-scatter sums the scaled partials over the ranks,
 * rank r keeping heads [r*H/N, (r+1)*H/N).  Concatenating the N slices of step 3
 * gives dcp_merge's O; step 1 gives its LSE.  The scaled partials can travel as
 * bf16, halving the reduce-scatter's bytes; each term then carries one bf16
 * rounding (relative 2^-9) before the fp32 sum.                              */
typedef enum { DCP_DTYPE_F32 = 0, DCP_DTYPE_BF16 = 1 } dcp_dtype_t;

/* Step 1.  lse_parts device fp32 [num_parts, batch, H] (the gathered LSE_r);
 * out_lse device fp32 [batch, H], written (-inf where every LSE_r is -inf).
 * Errors: INVALID_VALUE for num_parts < 1, negative sizes or NULL pointers.  */
dcp_status_t dcp_merge_lse(const float* lse_parts, int32_t num_parts, int32_t batch,
                           int32_t num_heads, float* out_lse, void* stream);

/* Step 2.  o_r device fp32 [batch, H, v_dim], lse_r and lse device fp32
 * [batch, H]; out device [batch, H, v_dim] of out_dtype (dcp_dtype_t), written
 * with exp(lse_r - lse) * o_r (0 where lse_r or lse is -inf).
 * Errors: INVALID_VALUE for v_dim not a multiple of 4, a bad dtype, NULL or
 * misaligned pointers.                                                        */
dcp_status_t dcp_rescale_partial(const float* o_r, const float* lse_r, const float* lse,
                                 int32_t batch, int32_t num_heads, int32_t v_dim,
                                 int32_t out_dtype, void* out, void* stream);

/* Step 3 for one rank.  scaled_parts device [num_parts, batch, H, v_dim] of
 * in_dtype (the N ranks' step-2 outputs, stacked); out device fp32
 * [batch, H / num_parts, v_dim], written with the sum over the parts of heads
 * [rank * H/num_parts, (rank+1) * H/num_parts).
 * Errors: INVALID_VALUE for H % num_parts != 0, rank outside [0, num_parts),
 * v_dim not a multiple of 4, a bad dtype, NULL or misaligned pointers.       */
dcp_status_t dcp_sum_head_slice(const void* scaled_parts, int32_t in_dtype, int32_t num_parts,
                                int32_t batch, int32_t num_heads, int32_t v_dim, int32_t rank,
                                float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DCP_H_ */
