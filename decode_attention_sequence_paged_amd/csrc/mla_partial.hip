// MLA partial decode attention over one rank's shard of a paged latent KV cache.
//
// What it computes (vLLM blog "Efficient Decode Context Parallelism with vLLM for
// Long Context Workloads", Sec. 4.1 "Compute" and Sec. 5.3 "MLA Backend"): every
// query head attends the rank's local latent rows; K is the whole 576-dim row and
// V its first 512 entries (the weight-absorbed form, where the query is already in
// the latent space).  Output: normalised partial O [B,H,512] and LSE [B,H].
//
// Design for gfx950:
//  * A work-group owns up to 64 query heads (4 waves x 16 heads) and a
//    token-balanced span of the rank's 32-token tiles; the span may cover the end
//    of one request, whole requests and the start of another.  Every latent row is
//    read from HBM once per head group and serves as both K and V.
//  * Tiles stream HBM -> LDS through a 4-stage ring of 16-byte direct-to-LDS copies
//    (no VGPR staging), issued three tiles ahead and continuing across request
//    boundaries.  LDS rows are padded to an odd stride of 73 16-byte slots, which
//    keeps the 16-row MFMA operand reads free of bank conflicts with affine
//    addresses; operand reads are software-pipelined a few MFMA steps ahead.
//  * Each wave owns 16 heads over the full 576 dims, so waves never exchange
//    partial scores: S^T = K Q^T (two 16x16x32 bf16 MFMA chains, tokens on the
//    rows, heads on the columns; the wave's 16 x 576 q slice lives in VGPRs), then
//    base-2 online softmax whose statistics are lane-local per head, then
//    O^T += V^T P^T where the S^T accumulator converted to bf16 is the B operand
//    and V^T comes from LDS through the transposing ds_read_b64_tr_b16.
//  * The running maximum moves only when a tile's maximum exceeds it by more than
//    kRescaleSlack (log2 units), so the 128-register O accumulator is rarely
//    rescaled; P stays <= 2^kRescaleSlack and the final LSE uses the same maximum,
//    so the result is unchanged.
#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {
namespace mla {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;            // 1152
constexpr int kChunks = kRowBytes / 16;        // 72 16-byte chunks per row
constexpr int kTile = 32;                      // tokens per tile
constexpr int kRowSlots = kChunks + 1;         // 73: odd LDS row stride in 16-byte slots
constexpr int kLdsRowBytes = kRowSlots * 16;   // 1168
constexpr int kTileSlots = kTile * kRowSlots;  // 2336
constexpr int kTileBytes = kTileSlots * 16;    // 37376
constexpr int kStages = 4;
constexpr int kPrefetch = 4;                   // LDS operand reads issued this many steps ahead
constexpr int kKSteps = kDqk / 32;             // 18 k-steps of 32 dims
constexpr int kVTiles = kDv / 16;              // 32 O^T tiles of 16 dims
constexpr float kRescaleSlack = 8.0f;
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// LDS byte offset of 16-byte chunk c of tile row `row`.  Rows are kRowSlots = 73
// slots apart: an odd stride puts the same chunk of 16 consecutive rows in 16
// different 4-bank groups (no conflicts), while every operand address stays
// affine in the chunk index (one base register plus an immediate offset).
__device__ __forceinline__ constexpr int chunk_off(int row, int c) { return row * kLdsRowBytes + c * 16; }

// Token (= LDS row) behind row i of a 16-row MFMA tile: rows 0..7 take the even
// tokens, rows 8..15 the odd ones.  The transposing read of V serves 32 lanes per
// LDS pass, i.e. lane groups q4 = {0,1} and {2,3}; with this order each pass reads 8
// rows of one parity, whose 32-byte pieces fall into disjoint banks at the 73-slot
// stride, and the 16 rows of an S^T tile stay distinct modulo 16 for the QK reads.
__device__ __forceinline__ constexpr int tile_row(int i) { return i < 8 ? 2 * i : 2 * (i - 8) + 1; }

template <int NW>
struct Cfg {
  static constexpr int kThreads = 64 * NW;
  static constexpr int kHeads = 16 * NW;
  // A tile is kTileSlots 16-byte slots written 64 at a time (one DMA instruction of a
  // wave); instruction j = k * NW + wave covers slots [64 j, 64 j + 64).  The slot
  // count is not a multiple of 64 * NW, so wave 0 issues one more (partly masked)
  // instruction than the others.
  static constexpr int kInstr = (kTileSlots + 63) / 64;        // 37
  static constexpr int kMainCopies = (kInstr - 1) / NW;        // full instructions per wave
  static constexpr int kTailLanes = kTileSlots - (kInstr - 1) * 64;  // 32 lanes of the last one
  static_assert((kInstr - 1) % NW == 0, "full copy instructions must split evenly over waves");
  static constexpr int kLoadsMax = kMainCopies + 1;            // wave 0
  static constexpr int kLoadsMin = kMainCopies;                // the other waves
  static_assert(kLoadsMax * (kStages - 2) < 64, "vmcnt range");
};

// Position in the span's sequence of (request, tile) pairs, 32-bit and division
// free inside the loop: the page of tile t is entry pk of the request's block-table
// row and the tile starts at token 32 * sub of that page (tpp tiles per page).
struct Cursor {
  int b, t, ntile, Lr, pk, sub;
  const int32_t* bt_row;
};

__device__ __forceinline__ void cursor_request(Cursor& c, const PartialParams& p, int b) {
  c.b = b;
  c.Lr = (int)part_local_len(p.part, b);
  c.ntile = (c.Lr + kTile - 1) / kTile;
  c.bt_row = p.block_table + (int64_t)b * p.max_blocks_per_seq;
}

__device__ __forceinline__ void cursor_set(Cursor& c, const PartialParams& p, int tpp, int b, int t) {
  cursor_request(c, p, b);
  c.t = t;
  c.pk = t / tpp;
  c.sub = t - c.pk * tpp;
}

// Advance to the next tile; only called while the span has tiles left, so a
// non-empty request follows whenever the current one is exhausted.
__device__ __forceinline__ void cursor_next(Cursor& c, const PartialParams& p, int tpp) {
  ++c.t;
  if (++c.sub == tpp) { c.sub = 0; ++c.pk; }
  if (c.t < c.ntile) return;
  do cursor_request(c, p, c.b + 1); while (c.ntile == 0 && c.b + 1 < p.part.batch);
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

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void mla_partial_kernel(PartialParams p) {
  using C = Cfg<NW>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kTileBytes];
  __shared__ int64_t s_scan[C::kThreads];
  __shared__ int64_t s_loc[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  int64_t w;
  int hg;
  block_to_span(p.part.num_parts, p.num_head_groups, &w, &hg);
  const bool write_prefix = (w == 0 && hg == 0);
  const SpanLoc loc = locate_span<C::kThreads>(p.part, w, write_prefix ? p.ws_prefix : nullptr,
                                               s_scan, s_loc);
  if (loc.start >= loc.end) return;
  const int total = (int)(loc.end - loc.start);
  const int tpp = p.block_size / kTile;                    // tiles per page
  const int64_t page_bytes = (int64_t)p.block_size * kRowBytes;
  // DMA copy instructions this wave issues per tile (wave 0 has the extra one).
  const bool extra_copy = wave == 0;

  const int H = p.num_q_heads;
  const int head = hg * C::kHeads + wave * 16 + l16;  // this lane's head (S^T column)
  const bool head_ok = head < H;
  DCP_LDS uint8_t* lds = (DCP_LDS uint8_t*)smem;

  // This lane's DMA copies: LDS slot (k * NW + wave) * 64 + lane of every tile
  // holds chunk (slot % 73) of row (slot / 73).  The 73rd slot of a row is never
  // read; its lane copies the row's last chunk again (same cache line) instead of
  // branching.  Every wave issues kMainCopies full instructions; wave 0 adds the
  // half-filled tail instruction, whose lanes past the tile are masked.
  int ld_row[C::kMainCopies];
  int ld_off[C::kMainCopies];
#pragma unroll
  for (int k = 0; k < C::kMainCopies; ++k) {
    const int s = (k * NW + wave) * 64 + lane;
    const int row = s / kRowSlots;
    const int c = s - row * kRowSlots;
    ld_row[k] = row;
    ld_off[k] = row * kRowBytes + (c < kChunks ? c : kChunks - 1) * 16;
  }
  int tail_row, tail_off;
  {
    const int s = C::kMainCopies * NW * 64 + lane;
    tail_row = s / kRowSlots;
    const int c = s - tail_row * kRowSlots;
    tail_off = tail_row * kRowBytes + (c < kChunks ? c : kChunks - 1) * 16;
  }
  const bool tail_lane = wave == 0 && lane < C::kTailLanes;

  Cursor lc, cc;
  cursor_set(lc, p, tpp, loc.b0, (int)loc.off0);
  cc = lc;

  // The page id is fetched (a scalar load the wave must wait for) only when the
  // loader enters a new page, i.e. once per tpp tiles.
  int32_t page = 0;
  bool page_stale = true;
  auto issue = [&](int stage) {
    if (lc.sub == 0 || page_stale) {
      page = clamp_page(ld_const(lc.bt_row + lc.pk), p.num_cache_blocks);
      page_stale = false;
    }
    const uint8_t* base = p.k_cache + page * page_bytes + lc.sub * (kTile * kRowBytes);
    DCP_LDS uint8_t* dst = lds + stage * kTileBytes;
    const int nvalid = lc.Lr - lc.t * kTile;
    if (nvalid >= kTile) {
#pragma unroll
      for (int k = 0; k < C::kMainCopies; ++k) dma16(base + ld_off[k], dst + (k * NW + wave) * 1024);
      if (tail_lane) dma16(base + tail_off, dst + C::kMainCopies * NW * 1024);
    } else {  // last tile of a request: rows past its end repeat its last row
#pragma unroll
      for (int k = 0; k < C::kMainCopies; ++k) {
        const int row = ld_row[k] < nvalid ? ld_row[k] : nvalid - 1;
        dma16(base + ld_off[k] - (ld_row[k] - row) * kRowBytes, dst + (k * NW + wave) * 1024);
      }
      const int row = tail_row < nvalid ? tail_row : nvalid - 1;
      if (tail_lane) dma16(base + tail_off - (tail_row - row) * kRowBytes, dst + C::kMainCopies * NW * 1024);
    }
  };

  // q[b, head, 32*s + 8*q4 .. +7]: the B operand of S^T = K Q^T for k-step s.
  bf16x8 qreg[kKSteps];
  auto load_q = [&](int b) {
    const uint16_t* qp = p.q + ((int64_t)b * H + (head_ok ? head : 0)) * kDqk + 8 * q4;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      bf16x8 v = *(const bf16x8*)(qp + 32 * s);
      qreg[s] = head_ok ? v : bf16x8{};
    }
    // The q slice is only an MFMA operand: keep it in accumulation registers so the
    // VGPRs stay free for the O accumulator and the operand prefetch ring.
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) asm volatile("" : "+a"(qreg[s]));
  };

  // prologue: up to kStages-1 tiles in flight
  int issued = 0;
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) {
    if (issued < total) {
      issue(s);
      if (++issued < total) cursor_next(lc, p, tpp);
    }
  }
  load_q(cc.b);

  f32x4 oacc[kVTiles];
#pragma unroll
  for (int m = 0; m < kVTiles; ++m) oacc[m] = f32x4{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  int piece_t0 = cc.t;  // first tile of the current piece inside request cc.b
  bool first_piece = true;
  int cstage = 0, istage = kStages - 1;

  for (int i = 0; i < total; ++i) {
    // Tile i has landed once at most the copies of the kStages-2 tiles issued after
    // it are outstanding (younger memory operations only make the wait stricter);
    // near the end of the span, drain everything.
    if (issued - i == kStages - 1) {
      if (extra_copy) wait_vmcnt_builtin<C::kLoadsMax * (kStages - 2)>();
      else wait_vmcnt_builtin<C::kLoadsMin * (kStages - 2)>();
    } else {
      wait_vmcnt_builtin<0>();
    }
    wg_barrier();
    if (issued < total) {
      issue(istage);
      istage = istage + 1 == kStages ? 0 : istage + 1;
      if (++issued < total) cursor_next(lc, p, tpp);
    }

    const DCP_LDS uint8_t* tb = lds + cstage * kTileBytes;
    cstage = cstage + 1 == kStages ? 0 : cstage + 1;
    const int nvalid = cc.Lr - cc.t * kTile;   // >= kTile for every tile but a request's last

    // ---- S^T [32 tokens x 16 heads] = K [32 x 576] Q^T, as two 16-token chains.
    // Operand reads run kPrefetch k-steps ahead of the MFMAs.
    f32x4 s0 = f32x4{}, s1 = f32x4{};
    {
      const DCP_LDS uint8_t* ka = tb + chunk_off(tile_row(l16), q4);   // + 64 * s (+ 16 rows)
      bf16x8 r0[kPrefetch], r1[kPrefetch];
#pragma unroll
      for (int s = 0; s < kPrefetch; ++s) {
        r0[s] = *(const DCP_LDS bf16x8*)(ka + 64 * s);
        r1[s] = *(const DCP_LDS bf16x8*)(ka + 16 * kLdsRowBytes + 64 * s);
      }
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) {
        const bf16x8 a0 = r0[s % kPrefetch];
        const bf16x8 a1 = r1[s % kPrefetch];
        if (s + kPrefetch < kKSteps) {
          r0[s % kPrefetch] = *(const DCP_LDS bf16x8*)(ka + 64 * (s + kPrefetch));
          r1[s % kPrefetch] = *(const DCP_LDS bf16x8*)(ka + 16 * kLdsRowBytes + 64 * (s + kPrefetch));
        }
        s0 = mfma16x16x32(a0, qreg[s], s0);
        s1 = mfma16x16x32(a1, qreg[s], s1);
      }
      // Keep 2*kPrefetch operand reads in flight: reads first, then (2 MFMA, 2 reads) ...
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPrefetch, 0);
#pragma unroll
      for (int s = 0; s < kKSteps - kPrefetch; ++s) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * kPrefetch, 0);
    }

    // ---- online softmax (base 2).  Lane: head l16, tokens 16*(j/4) + tile_row(4*q4 + j%4).
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (j < 4 ? s0[j] : s1[j - 4]) * p.scale_log2;
    if (nvalid < kTile) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (16 * (j >> 2) + tile_row(4 * q4 + (j & 3)) >= nvalid) x[j] = -INFINITY;
    }
    float mloc = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                       fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mloc = max_over_groups(mloc);
    const float m_new = mloc > m_run + kRescaleSlack ? mloc : m_run;
    const float alpha = fast_exp2(m_run - m_new);
    float lsum = 0.f;
    bf16x8 pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float pr = fast_exp2(x[j] - m_new);
      lsum += pr;
      pb[j] = (__bf16)pr;
    }
    lsum = sum_over_groups(lsum);
    l_run = l_run * alpha + lsum;
    if (__any(m_new != m_run)) {
#pragma unroll
      for (int m = 0; m < kVTiles; ++m) oacc[m] *= alpha;
    }
    m_run = m_new;

    // ---- O^T [512 dims x 16 heads] += V^T [512 x 32 tokens] P^T [32 x 16].
    // Source lane l16 of each 16-lane group addresses row tile_row(4*q4 + l16/4) (and
    // +16), dims 16m + 4*(l16%4) .. +3, i.e. chunk 2m + (l16%4)/2, half (l16%2); lane
    // i then holds dim 16m + i of the tokens P's element j stands for.
    {
      const DCP_LDS uint8_t* va =
          tb + chunk_off(tile_row(4 * q4 + (l16 >> 2)), (l16 & 3) >> 1) + (l16 & 1) * 8;
      u32x2 v1[kPrefetch], v2[kPrefetch];
#pragma unroll
      for (int m = 0; m < kPrefetch; ++m) {
        v1[m] = lds_read_tr16(va + 32 * m);
        v2[m] = lds_read_tr16(va + 16 * kLdsRowBytes + 32 * m);
      }
#pragma unroll
      for (int m = 0; m < kVTiles; ++m) {
        const bf16x8 a = join_tr16(v1[m % kPrefetch], v2[m % kPrefetch]);
        if (m + kPrefetch < kVTiles) {
          v1[m % kPrefetch] = lds_read_tr16(va + 32 * (m + kPrefetch));
          v2[m % kPrefetch] = lds_read_tr16(va + 16 * kLdsRowBytes + 32 * (m + kPrefetch));
        }
        oacc[m] = mfma16x16x32(a, pb, oacc[m]);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPrefetch, 1);
#pragma unroll
      for (int m = 0; m < kVTiles - kPrefetch; ++m) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPrefetch, 1);
    }

    // ---- end of a request piece: normalise and store, then move to the next request
    const bool last_of_req = cc.t == cc.ntile - 1;
    if (last_of_req || i == total - 1) {
      const bool whole = piece_t0 == 0 && last_of_req;
      if (head_ok) {
        const float inv = 1.0f / l_run;
        const int64_t slot = 2 * w + (first_piece ? 0 : 1);
        float* orow = whole ? p.out_o + ((int64_t)cc.b * H + head) * kDv
                            : p.ws_o + (slot * H + head) * kDv;
#pragma unroll
        for (int m = 0; m < kVTiles; ++m) *(f32x4*)(orow + 16 * m + 4 * q4) = oacc[m] * inv;
        if (q4 == 0) {
          const float lse = (m_run + fast_log2(l_run)) * kLn2;
          if (whole) p.out_lse[(int64_t)cc.b * H + head] = lse;
          else p.ws_lse[slot * H + head] = lse;
        }
      }
      if (i + 1 < total) {
        cursor_next(cc, p, tpp);
        piece_t0 = 0;
        first_piece = false;
        load_q(cc.b);
        wait_vmcnt_builtin<0>();
#pragma unroll
        for (int m = 0; m < kVTiles; ++m) oacc[m] = f32x4{};
        m_run = -INFINITY;
        l_run = 0.f;
      }
    } else {
      cursor_next(cc, p, tpp);
    }
  }
}

}  // namespace mla

int mla_heads_per_group(int num_q_heads) { return num_q_heads <= 32 ? 32 : 64; }

hipError_t launch_mla_partial(const PartialParams& p, hipStream_t stream) {
  const int grid = p.part.num_parts * p.num_head_groups;
  if (mla_heads_per_group(p.num_q_heads) == 32)
    hipLaunchKernelGGL(mla::mla_partial_kernel<2>, dim3(grid), dim3(128), 0, stream, p);
  else
    hipLaunchKernelGGL(mla::mla_partial_kernel<4>, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dcp
