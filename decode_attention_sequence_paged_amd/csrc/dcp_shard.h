// Sequence-dimension shard map of a request's KV cache (host and device).
//
// Decode Context Parallelism keeps the KV cache of every request split along
// the sequence dimension, each rank holding a subset of the token positions
// (vLLM blog "Efficient Decode Context Parallelism with vLLM for Long Context
// Workloads", Sec. 4 and Sec. 2.2).  Positions are dealt to the N ranks
// round-robin in runs of I consecutive tokens, I being the KV-cache interleave
// size of the vLLM-Ascend "Decode Context Parallel Guide" (Constraints).  A rank
// stores its tokens densely in ascending global order.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define DCP_HD __host__ __device__ __forceinline__
#else
#define DCP_HD static inline
#endif

// Rank that holds global position t.
DCP_HD int32_t dcp_owner(int64_t t, int32_t N, int32_t I) { return (int32_t)((t / I) % N); }

// Index of global position t inside its owner's dense local order.
DCP_HD int64_t dcp_local_index(int64_t t, int32_t N, int32_t I) {
  return (t / ((int64_t)N * I)) * I + t % I;
}

// Global position of local index j on rank r (inverse of dcp_local_index).
DCP_HD int64_t dcp_global_index(int64_t j, int32_t N, int32_t I, int32_t r) {
  return ((j / I) * N + r) * (int64_t)I + j % I;
}

// Number of the L positions of a request that rank r holds: every complete round of
// N*I positions gives each rank I of them; the positions of the last, incomplete
// round go to the lowest ranks first, I at a time.
DCP_HD int64_t dcp_local_len(int64_t L, int32_t N, int32_t I, int32_t r) {
  if (L <= 0) return 0;
  const int64_t round = (int64_t)N * I;
  const int64_t full = L / round;
  int64_t extra = (L - full * round) - (int64_t)r * I;
  extra = extra < 0 ? 0 : (extra > I ? (int64_t)I : extra);
  return full * I + extra;
}
