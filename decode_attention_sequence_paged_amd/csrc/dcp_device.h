// Device-side helpers shared by the decode-attention kernels (gfx950 / CDNA4).
#pragma once
#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcp_params.h"
#include "dcp_partition.h"
#include "dcp_shard.h"

#define DCP_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((__vector_size__(8)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

namespace dcp {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Work-group barrier without a memory fence: the kernels order their LDS traffic
// with explicit s_waitcnt, so the fence __syncthreads() adds (which also drains
// every outstanding global load) is not wanted.  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The same wait as a compiler builtin, so the compiler's own wait-count tracking
// sees it (it then knows every older load, e.g. of the query slice, has landed).
template <int N>
__device__ __forceinline__ void wait_vmcnt_builtin() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt immediate: vmcnt[3:0], expcnt[6:4] = 7 (no wait), lgkmcnt[11:8] = 15
  // (no wait), vmcnt[5:4] in bits [15:14].
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// 16-byte asynchronous global -> LDS copy.  Lane i's 16 bytes land at
// lds_wave_base + 16 * i (lds_wave_base must be wave-uniform).
__device__ __forceinline__ void dma16(const void* gsrc, DCP_LDS void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_wave_base, 16, 0, 0);
}

// LDS transpose read of four 16-bit values.  Inside each group of 16 lanes, lane
// i receives element (i % 4) of the 8-byte pieces addressed by lanes
// (i / 4) + 4e, e = 0..3.  If source lane s of the group addresses row r0 + s/4,
// columns c0 + 4(s%4) .. +3 of a row-major bf16 matrix, lane i obtains column
// c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ u32x2 lds_read_tr16(const DCP_LDS void* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((DCP_LDS i16x4*)p));
}

// Joins two transposed 4-element reads into one 8-element MFMA operand.  The
// values are moved as whole dwords: assembling the bf16 vector element by element
// from the 16-bit lanes of the read result is mis-packed by this compiler (it
// duplicates element 0).
__device__ __forceinline__ bf16x8 join_tr16(u32x2 lo, u32x2 hi) {
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Softmax weights as MFMA operands.  A bf16 operand keeps 8 significant bits, so a
// weight rounded to bf16 moves by up to 2^-8 of itself; when a few tokens carry most
// of a row's weight (a short request) that reaches the output as up to about
// 2^-8 |V|, close to the 5e-3 accuracy bound.  The P.V products therefore take P as
// two bf16 operands accumulated into the same O, hi = bf16(P) and lo = P - hi
// (|lo| <= 2^-8 P), so that the weights enter with about 16 significant bits.  The
// row sum l is accumulated from the fp32 P.
//
// The low parts only matter for weights that end up a sizeable share of their row.
// A tile takes them if its request has at most kLowAllTokens local tokens, or if some
// weight in it exceeds kLowShare of its row's running sum (every first tile of a
// piece, and later tiles that hold a dominant token).  The weights of the other
// tiles are each below kLowShare of the row's final sum and spread over more than
// kLowAllTokens tokens, so their bf16 rounding errors average out (below about 7e-4
// with 64 heads of 512 dims).  In long rows few tiles qualify, so the extra MFMAs
// cost little there.
constexpr float kLowShare = 0.25f;
constexpr int kLowAllTokens = 256;
__device__ __forceinline__ __bf16 bf16_low_part(float x, __bf16 hi) { return (__bf16)(x - (float)hi); }

// Low parts handed from one wave to another through LDS are coded compactly, as fp8
// (OCP e4m3: 4 significant bits, finite up to 448) of lo * 2^8.  P <= 2^8 (the lazy
// rescale's slack) keeps the code at most 2^8; a lo below 2^-18 (a weight below about
// 2^-10 of the row maximum) codes to 0 and leaves that weight at bf16 precision.
// Eight codes per lane: codes 2k and 2k+1 in 16-bit half k % 2 of word k / 2; the
// decode multiplies by 2^-8 on its way to bf16.
constexpr float kLowScale = 256.f;
__device__ __forceinline__ u32x2 code_low_parts(const float lo[8]) {
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(lo[0] * kLowScale, lo[1] * kLowScale, 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(lo[2] * kLowScale, lo[3] * kLowScale, w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(lo[4] * kLowScale, lo[5] * kLowScale, 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(lo[6] * kLowScale, lo[7] * kLowScale, w1, true);
  return u32x2{(unsigned)w0, (unsigned)w1};
}
__device__ __forceinline__ bf16x8 decode_low_parts(u32x2 w) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  constexpr float kInv = 1.f / kLowScale;
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[0], kInv, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[0], kInv, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[1], kInv, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[1], kInv, true);
  // moved as whole dwords (see join_tr16)
  return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                          __builtin_bit_cast(unsigned, c), __builtin_bit_cast(unsigned, d)});
}

__device__ __forceinline__ int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Load through the constant address space: the data is read-only for the whole
// kernel, so a wave-uniform address becomes a scalar load (counted by lgkmcnt, not
// by vmcnt, so it never waits behind the in-flight direct-to-LDS tile copies).
template <class T>
__device__ __forceinline__ T ld_const(const T* ptr) {
  return *(const __attribute__((address_space(4))) T*)ptr;
}

// Page id of a block-table entry, clamped into the pool (an entry outside [0, num_blocks)
// reads page 0, so no copy leaves the pool); such an entry sets `bad`.
__device__ __forceinline__ int32_t checked_page(int32_t page, int64_t num_blocks, bool& bad) {
  const bool out = page < 0 || (int64_t)page >= num_blocks;
  bad = bad || out;
  return out ? 0 : page;
}

// Bit values of the device error word (the same as dcp_device_error_t in dcp.h).
constexpr uint32_t kErrPageId = 1u, kErrTableShort = 2u, kErrNegLength = 4u;

// Adds bits to the device error word (one lane of a wave calls it; vector atomic).
__device__ __forceinline__ void report_error(uint32_t* err, uint32_t bits) {
  __hip_atomic_fetch_or(err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ work partitions
//
// How a rank's tiles are cut into spans of equal work, and which workspace slot each
// request piece takes: dcp_partition.h (shared with the host tests).

// Local length of request b actually processed (clamped to what its block table row holds).
__device__ __forceinline__ int64_t part_local_len(const PartitionArgs& a, int b) {
  int64_t L = (int64_t)ld_const(a.seq_lens + b) - a.len_offset;
  int64_t lr = dcp_local_len(L < 0 ? 0 : L, a.num_ranks, a.interleave, a.rank);
  const int64_t cap = (int64_t)a.max_blocks_per_seq * a.block_size;
  return lr < cap ? lr : cap;
}

__device__ __forceinline__ int64_t part_tiles(const PartitionArgs& a, int b) {
  return (part_local_len(a, b) + a.tile - 1) / a.tile;
}

constexpr int kCountBits = 17;  // packed scan value: tiles << kCountBits | requests with tiles

struct SpanLoc {
  int64_t total;   // TT
  int64_t start;   // first tile of the span
  int64_t end;     // one past its last tile
  int32_t b0;      // request of the first tile
  int64_t off0;    // tile offset of the first tile inside request b0
};

// Block-cooperative: every thread of the block gets the location of span w.  If
// prefix_out is non-null, the block also writes each request's first tile index
// (prefix_out[b], the total at prefix_out[B]), weighted position (prefix_out[B + 1 +
// b], the weighted total at prefix_out[2 B + 1]) and the spans of its first and last
// tiles (prefix_out[2 B + 2 + b] = w_first << 32 | w_last; 0 for a request without
// tiles), so that the split reduce need not repeat the partition arithmetic, and adds to
// *err_word the bits of the lengths it had to clamp.  s_scan must hold blockDim.x / 64
// int64 values; s_loc four int64 values.
template <int NT>
__device__ __forceinline__ SpanLoc locate_span(const PartitionArgs& a, int64_t w, int64_t* prefix_out,
                               uint32_t* err_word, int64_t* s_scan, int64_t* s_loc) {
  constexpr int64_t kCountMask = (int64_t(1) << kCountBits) - 1;
  const int tid = threadIdx.x;
  const int per = (a.batch + NT - 1) / NT;
  const int b_lo = tid * per;
  const int b_hi = min(a.batch, b_lo + per);
  int64_t sum = 0;
  for (int b = b_lo; b < b_hi; ++b) {
    const int64_t n = part_tiles(a, b);
    sum += (n << kCountBits) | (n > 0 ? 1 : 0);
  }
  // Inclusive scan of the per-thread sums: within each wave by shuffles, then the
  // wave totals through LDS (one barrier instead of two per doubling step).
  static_assert(NT % 64 == 0 && NT / 64 <= 16, "block shape");
  const int lane = tid & 63;
  int64_t incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t u = __shfl_up(incl, d, 64);
    if (lane >= d) incl += u;
  }
  if (lane == 63) s_scan[tid >> 6] = incl;
  if (tid == 0) { s_loc[0] = -1; s_loc[1] = 0; s_loc[2] = 0; s_loc[3] = 0; }
  __syncthreads();
  int64_t tot = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    const int64_t wt = s_scan[k];
    if (k < (tid >> 6)) incl += wt;
    tot += wt;
  }
  const int64_t excl = incl - sum;
  const int64_t A = a.req_weight;
  const int64_t TT = tot >> kCountBits;
  const int64_t WT = TT + A * (tot & kCountMask);
  const int64_t x0 = dcp_span_start(w, WT, a.num_parts, a.xcd_weighted);
  const int64_t x1 = dcp_span_start(w + 1, WT, a.num_parts, a.xcd_weighted);
  // Walk this thread's requests; the one whose weighted range holds x0 (x1) gives
  // the span's first (end) tile.
  int64_t F = excl >> kCountBits;
  int64_t WP = F + A * (excl & kCountMask);
  uint32_t err = 0;
  for (int b = b_lo; b < b_hi; ++b) {
    const int64_t n = part_tiles(a, b);
    if (prefix_out) {
      // device-resident lengths the kernels had to clamp (checked by one work-group)
      const int32_t raw = ld_const(a.seq_lens + b);
      if (raw < 0) err |= kErrNegLength;
      const int64_t Lr = dcp_local_len(raw - (int64_t)a.len_offset, a.num_ranks, a.interleave, a.rank);
      if (Lr > (int64_t)a.max_blocks_per_seq * a.block_size) err |= kErrTableShort;
      prefix_out[b] = F;
      prefix_out[a.batch + 1 + b] = WP;
      int64_t span_range = 0;
      if (n > 0) {
        const int64_t wf = dcp_span_of(WP + A, WT, a.num_parts, a.xcd_weighted);
        const int64_t wl = dcp_span_of(WP + A + n - 1, WT, a.num_parts, a.xcd_weighted);
        span_range = (wf << 32) | wl;
      }
      prefix_out[2 * a.batch + 2 + b] = span_range;
    }
    if (n > 0) {
      const int64_t wend = WP + A + n;
      if (x0 < x1 && WP <= x0 && x0 < wend) {
        const int64_t start = dcp_span_cut(x0, WP, A, F);
        s_loc[0] = b; s_loc[1] = start - F; s_loc[2] = start;
      }
      if (WP <= x1 && x1 < wend) s_loc[3] = dcp_span_cut(x1, WP, A, F);
      F += n;
      WP = wend;
    }
  }
  if (prefix_out && tid == NT - 1) { prefix_out[a.batch] = TT; prefix_out[2 * a.batch + 1] = WT; }
  if (err) report_error(err_word, err);
  __syncthreads();
  // Every lane read the same LDS values; say so, so that what the kernels derive from
  // the span (loop bounds, page bases) stays in scalar registers.
  SpanLoc loc;
  loc.total = uniform64(TT);
  loc.b0 = uniform((int32_t)s_loc[0]);
  loc.off0 = uniform64(s_loc[1]);
  loc.start = uniform64(x0 < x1 ? s_loc[2] : 0);
  loc.end = uniform64(x0 < x1 ? (x1 >= WT ? TT : s_loc[3]) : 0);
  __syncthreads();  // s_loc / s_scan may be reused after this
  return loc;
}

// Split the flat block index into (span, head group).  Consecutive dispatches go
// round-robin over the 8 XCDs, so blocks x and x + 8 share an XCD; with several
// head groups the groups of one span are placed 8 apart, so they read the same
// pages through the same L2 at about the same time, and each XCD takes a contiguous
// eighth of the spans (measured 2-5% faster than spans dealt round-robin over the XCDs
// for the 1M-token request; with one head group the round-robin order is kept, as
// the contiguous one was no faster there).
__device__ __forceinline__ void block_to_span(int num_parts, int num_groups, int64_t* w, int* g) {
  const int x = blockIdx.x;
  if (num_groups == 1) { *w = x; *g = 0; return; }
  if (num_parts % 8 == 0) {
    const int xcd = x % 8, k = x / 8;
    *w = (int64_t)xcd * (num_parts / 8) + k / num_groups;
    *g = k % num_groups;
  } else {
    *w = x / num_groups;
    *g = x % num_groups;
  }
}



constexpr int kTileTokens = 32;  // tokens per streamed tile (both kernels)

// ------------------------------------------------------------------ tile cursor
//
// Position in a span's sequence of (request, tile) pairs, 32-bit and division free
// inside the loops: the page of tile t is entry pk of the request's block-table row
// and the tile starts at token T * sub of that page (tpp tiles of T tokens per page;
// T = kTileTokens unless a kernel streams other tiles).
struct Cursor {
  int b, t, ntile, Lr, pk, sub;
  int Lg;  // the request's global length
  const int32_t* bt_row;
};

template <int T = kTileTokens>
__device__ __forceinline__ void cursor_request(Cursor& c, const PartialParams& p, int b) {
  c.b = b;
  const int32_t L = ld_const(p.part.seq_lens + b) - p.part.len_offset;
  c.Lg = L < 0 ? 0 : L;
  c.Lr = (int)part_local_len(p.part, b);
  c.ntile = (c.Lr + T - 1) / T;
  c.bt_row = p.block_table + (int64_t)b * p.max_blocks_per_seq;
}

template <int T = kTileTokens>
__device__ __forceinline__ void cursor_set(Cursor& c, const PartialParams& p, int tpp, int b, int t) {
  cursor_request<T>(c, p, b);
  c.t = t;
  c.pk = t / tpp;
  c.sub = t - c.pk * tpp;
}

// Advance to the next tile; only called while the span has tiles left, so a
// non-empty request follows whenever the current one is exhausted.
template <int T = kTileTokens>
__device__ __forceinline__ void cursor_next(Cursor& c, const PartialParams& p, int tpp) {
  ++c.t;
  if (++c.sub == tpp) { c.sub = 0; ++c.pk; }
  if (c.t < c.ntile) return;
  do cursor_request<T>(c, p, c.b + 1); while (c.ntile == 0 && c.b + 1 < p.part.batch);
  c.t = c.pk = c.sub = 0;
}

// Cross-lane reductions over the lanes l, l^16, l^32, l^48 (one head's four lane
// groups) with the gfx950 row-swap permutes: applying the operation to the two
// outputs of a swap of x with itself combines x with its partner lane.
__device__ __forceinline__ float max_over_groups(float x) {
  auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}
__device__ __forceinline__ float sum_over_groups(float x) {
  auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// Causal mask of multi-token decode queries: the q_len queries are the request's last
// q_len positions, and query i (score row `row`, i = row / heads_per_token) sees the
// global positions <= Lg - q_len + i.  Masks this lane's eight scores (tokens 4 q4 + e
// and 16 + 4 q4 + e of the tile at cursor `cur`).  The local tokens every query sees
// (global position <= Lg - q_len) are the first dcp_local_len(Lg - q_len + 1) of the
// request; that count is computed once per request (CausalFrom), so a tile before it is
// left alone after one wave-uniform compare.
struct CausalFrom {
  int b = -1;
  int64_t from = 0;  // local tokens of request b that every query sees
};

__device__ __forceinline__ void causal_mask(const PartialParams& p, const Cursor& cur, int nvalid,
                                            int row, int q4, f32x4& s0, f32x4& s1, CausalFrom& cf) {
  if (p.q_len <= 1) return;
  const int N = p.part.num_ranks, I = p.part.interleave, r = p.part.rank;
  const int64_t lim0 = (int64_t)cur.Lg - p.q_len;
  if (cur.b != cf.b) {
    cf.b = cur.b;
    cf.from = dcp_local_len(lim0 + 1, N, I, r);
  }
  const int64_t j0 = (int64_t)cur.t * kTileTokens;
  const int64_t last = j0 + (nvalid < kTileTokens ? nvalid : kTileTokens) - 1;
  if (last < cf.from) return;
  const int64_t lim = lim0 + row / p.heads_per_token;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (dcp_global_index(j0 + 4 * q4 + e, N, I, r) > lim) s0[e] = -INFINITY;
    if (dcp_global_index(j0 + 16 + 4 * q4 + e, N, I, r) > lim) s1[e] = -INFINITY;
  }
}

// s_waitcnt lgkmcnt(0) as a builtin, so the compiler's own wait counting knows every
// earlier LDS access and scalar load has completed.
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ uint32_t lds_addr(const DCP_LDS void* p) { return (uint32_t)(uintptr_t)p; }

// ------------------------------------------------------------------ LDS and copy asm
// 16-byte global -> LDS copy: lane i's bytes from base + off land at lds_dst + 16 i.
// Also asm, for the same reason: the compiler then neither counts these copies nor
// drains them before LDS accesses; the kernel's explicit vmcnt waits order them.
// No memory clobber: the copies only write a stage that no access in flight
// touches, so LDS reads may be scheduled freely around them.
// kStream marks the loads non-temporal (nt): for pages that only this work-group
// reads, streaming them past the caches raised the attained HBM bandwidth by 7-11%
// (measured); pages that the head groups of a span share through their XCD's L2 are
// read with the default policy, which keeps them there for the partner.
// `base` must be wave-uniform; it is passed through readfirstlane so that it stays in scalar
// registers whatever the compiler concludes about the control flow around the call.
template <bool kStream>
__device__ __forceinline__ void copy16(const uint8_t* base, uint32_t off, uint32_t lds_dst) {
  const uint8_t* sbase = (const uint8_t*)uniform64((int64_t)base);
  if constexpr (kStream)
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" : : "v"(off), "s"(sbase), "{m0}"(lds_dst));
  else
    asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(sbase), "{m0}"(lds_dst));
}
__device__ __forceinline__ void zero_lds16(uint32_t addr) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(u32x4{0u, 0u, 0u, 0u}) : "memory");
}

}  // namespace dcp
