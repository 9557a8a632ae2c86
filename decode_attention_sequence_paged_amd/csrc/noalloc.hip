// dcp_decode_partial without a caller workspace, for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops, harnesses that forbid allocation):
// the same validation and kernels as dcp_decode_partial, with the workspace taken from a
// static device array of this library.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/dcp.h"
#include "dcp_internal.h"

namespace {

// 72 MiB: the workspace of every supported single-token shape at the default work
// partitions, for up to 65,536 requests.  The split pieces take at most 64 MiB (2 slots x
// 256 partitions x 64 heads x 512 dims x 4 bytes; 128 or more heads use proportionally
// fewer partitions per head group), the partition prefix 1.5 MiB.
constexpr size_t kScratchBytes = size_t(72) << 20;
constexpr int kMaxDevices = 64;

// One copy per device, held until the process ends.  In host code `scratch` names a
// host-side stand-in: kernels get the device address that hipGetSymbolAddress returns.
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once known

// Device address of this device's scratch.  The first call on a device looks it up and
// zeroes the array on `stream` (the device error word in its header starts clear).
dcp_status_t current_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DCP_ERROR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DCP_ERROR_HIP;
    if (dcp::launch_zero_fill(ptr, kScratchBytes, stream) != hipSuccess) return DCP_ERROR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DCP_SUCCESS;
}

}  // namespace

extern "C" dcp_status_t dcp_decode_partial_noalloc(const dcp_attn_desc_t* desc, const void* q,
                                                   const void* k_cache, const void* v_cache,
                                                   int64_t num_cache_blocks, const int32_t* block_table,
                                                   int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                                   int32_t batch, int32_t rank, int32_t num_ranks,
                                                   int32_t interleave, int32_t num_partitions,
                                                   float* out_o, float* out_lse, void* stream) {
  // Argument checks first, with no workspace: every error but the workspace's is final.
  dcp_status_t st = dcp_decode_partial(desc, q, k_cache, v_cache, num_cache_blocks, block_table,
                                       max_blocks_per_seq, seq_lens, batch, rank, num_ranks, interleave,
                                       num_partitions, nullptr, 0, out_o, out_lse, stream);
  if (st != DCP_ERROR_WORKSPACE) return st;
  if (dcp_decode_workspace_size(desc, batch, num_partitions) > kScratchBytes) return DCP_ERROR_WORKSPACE;
  void* ws = nullptr;
  st = current_scratch((hipStream_t)stream, &ws);
  if (st != DCP_SUCCESS) return st;
  return dcp_decode_partial(desc, q, k_cache, v_cache, num_cache_blocks, block_table, max_blocks_per_seq,
                            seq_lens, batch, rank, num_ranks, interleave, num_partitions, ws, kScratchBytes,
                            out_o, out_lse, stream);
}
