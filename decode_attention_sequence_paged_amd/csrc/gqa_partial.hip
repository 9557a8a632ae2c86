// GQA partial decode attention over one rank's shard of a paged K/V cache.
//
// What it computes (vLLM blog "Efficient Decode Context Parallelism with vLLM for
// Long Context Workloads", Sec. 4.1 "Compute" and Sec. 5.4 "GQA Backend"): each KV
// head is shared by its group of G = H / Hkv query heads (query head h reads KV
// head h / G).  Output: normalised partial O [B,H,128] and LSE [B,H] over the
// rank's tokens.
//
// Design for gfx950:
//  * One wave per KV head, up to 4 KV heads per work-group, so a token's K slice and
//    V slice of the group are contiguous (256 bytes per head).  The work-group owns a
//    span of the rank's 16-token tiles of equal work (same partitioning as the MLA
//    kernels).
//  * The loop does little arithmetic per byte (16 query heads per KV head), so what
//    sets its speed is how many bytes are in flight while memory latency runs under
//    a full HBM stream.  Tiles are 16 tokens (K part + V part, 2 x 16 rows x 256 B per
//    head: 32 KB for 4 KV heads) in a 4-stage ring of 16-byte direct-to-LDS copies,
//    so three tiles are in flight while one is computed.  A 16-token tile never
//    crosses a page (page sizes are multiples of 16), so a copy's source is one
//    scalar page base per tile plus a 32-bit lane offset computed once.
//  * Rows are XOR-swizzled inside each head's 16 chunks (x(r) = 2 (r & 7)): with the
//    gfx950 pass grouping of ds_read_b128 (lane quads of even / odd popcount within
//    each half-wave) the K operand reads hit 16 distinct bank groups per pass, and
//    the transposing V read stays at two lanes per bank.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (the 16 tokens on the rows, the KV
//    head's query heads on the columns); O^T += V^T P^T on v_mfma_f32_16x16x16_bf16,
//    whose A operand (16 dims x 4 tokens per lane quad) is exactly what one
//    ds_read_b64_tr_b16 returns and whose B operand is the S^T layout; base-2 online
//    softmax with the same lazy rescale as the MLA kernels.
//  * Rows of a request's partial last tile past its end are copied from the page
//    (always inside the pool) and made inert: scores -inf, V part zeroed in LDS.
//    Finished pieces are stored after the next barrier, ahead of the next copies.
//  * Multi-token decode queries (blog Sec. 6): QB query tokens of a request (QB = 1, 2
//    or 4) go on QB consecutive MFMA column blocks of the same KV head, so a pass
//    streams the pages once for all of them: every K and V^T operand read feeds QB
//    MFMAs.  Query token i sees the global positions <= L - q_len + i; the pass's
//    partition covers its newest token's positions and the older tokens' columns
//    mask the few newest positions they may not see.
//  * P enters the P.V MFMAs as its bf16 high part and, in the tiles where a weight is
//    a sizeable share of its row, also as its bf16 low part (bf16_low_part in
//    dcp_device.h).
#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {
namespace gqa {

constexpr int kD = 128;
constexpr int kHeadBytes = kD * 2;  // 256
constexpr int kTile = 16;           // tokens per tile
constexpr int kRingBytes = 128 * 1024;
constexpr float kRescaleSlack = 8.0f;
static_assert(kGqaTile == kTile, "tile size");

template <int KVW>
struct Cfg {
  static constexpr int kThreads = 64 * KVW;
  static constexpr int kRowBytes = KVW * kHeadBytes;        // one token's slice of the group
  static constexpr int kChunks = kRowBytes / 16;            // 16 * KVW
  static constexpr int kHalfBytes = kTile * kRowBytes;      // K (or V) part of a stage
  static constexpr int kStageBytes = 2 * kHalfBytes;
  static constexpr int kStages = kRingBytes / kStageBytes > 4 ? 4 : kRingBytes / kStageBytes;
  static constexpr int kCopies = kTile * kChunks / kThreads;  // per wave: 4 for K, 4 for V
  static constexpr int kTileOps = 2 * kCopies;                // copy instructions per wave and tile
  static_assert(kCopies == 4, "copy geometry");
  static_assert(kStages >= 3 && (kStages - 2) * kTileOps < 64, "ring depth");
};

// Chunk c (0 .. 16*KVW-1) of tile row r sits at position c ^ x(r) of the row; the
// XOR stays inside the head's 16 chunks.
__device__ __forceinline__ constexpr int row_swz(int r) { return 2 * (r & 7); }

__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                   __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

template <int KVW, int QB>
__global__ __launch_bounds__(64 * KVW, 1) void gqa_partial_kernel(PartialParams p) {
  static_assert(QB == 1 || QB == 2 || QB == 4, "query tokens per pass");
  using C = Cfg<KVW>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kStages * C::kStageBytes];
  __shared__ int64_t s_scan[C::kThreads];
  __shared__ int64_t s_loc[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int l16 = lane & 15;
  const int q4 = lane >> 4;  // 0..3

  int64_t w;
  int hg;
  block_to_span(p.part.num_parts, p.num_head_groups, &w, &hg);
  const bool write_prefix = (w == 0 && hg == 0);
  const SpanLoc loc = locate_span<C::kThreads>(p.part, w, write_prefix ? p.ws_prefix : nullptr,
                                               p.ws_err, s_scan, s_loc);
  if (loc.start >= loc.end) return;
  const int total = (int)(loc.end - loc.start);
  const int bs = p.block_size;
  const int tpp = bs / kTile;  // tiles per page

  const int H = p.num_q_heads;
  const int Hkv = p.num_kv_heads;
  const int G = H / Hkv;
  const int g0 = hg * KVW;             // first KV head of the work-group
  const int g = g0 + wave;             // this wave's KV head
  const bool head_ok = l16 < G;
  const int head = g * G + (head_ok ? l16 : 0);  // this lane's query head (S^T column)
  const int64_t row_stride = (int64_t)Hkv * kHeadBytes;  // bytes between token rows in the pool
  const int rows = QB * H;  // piece rows of a request: query token c's head h is row c H + h
  const int64_t page_bytes = (int64_t)bs * row_stride;
  DCP_LDS uint8_t* lds = (DCP_LDS uint8_t*)smem;

  // This lane's copies: LDS slot s = (k * KVW + wave) * 64 + lane of a tile half is
  // position s % kChunks of row s / kChunks, which holds chunk (pos ^ x(row)).
  uint32_t ld_off[C::kCopies];
#pragma unroll
  for (int k = 0; k < C::kCopies; ++k) {
    const int s = (k * KVW + wave) * 64 + lane;
    const int row = s / C::kChunks;
    const int pos = s - row * C::kChunks;
    ld_off[k] = (uint32_t)(row * row_stride + g0 * kHeadBytes + (pos ^ row_swz(row)) * 16);
  }

  // Operand offsets inside a stage half.  K: row l16, chunk 16 wave + 4 s + q4 of
  // k-step s -> ka[s].  V^T of dim block m: row 4 q4 + l16 / 4, dims 16 m + 4 (l16 % 4)
  // .. +3, i.e. chunk 16 wave + 2 m + (l16 % 4) / 2, byte half l16 % 2 -> va[m]; the
  // transposing read then gives lane (q4, l16) dim 16 m + l16 of tokens 4 q4 .. +3.
  uint32_t ka[4], va[8];
  {
    const int r = l16;
    const int x = row_swz(r);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      ka[s] = (uint32_t)(r * C::kRowBytes + wave * kHeadBytes + ((4 * s + q4) ^ x) * 16);
  }
  {
    const int r = 4 * q4 + (l16 >> 2);
    const int x = row_swz(r);
    const int h = (l16 & 3) >> 1;
#pragma unroll
    for (int m = 0; m < 8; ++m)
      va[m] = (uint32_t)(r * C::kRowBytes + wave * kHeadBytes + ((2 * m + h) ^ x) * 16 + 8 * (l16 & 1));
  }

  Cursor lc, cc;
  cursor_set<kTile>(lc, p, tpp, loc.b0, (int)loc.off0);
  cc = lc;

  // Copy source of the loader's tile (the pool byte offset of its first row).  Past
  // the end of the span the loader stays on the last tile, which is copied again
  // into a stage no wave reads.
  int lc_left = total;
  int64_t src = 0;
  bool bad_page = false;
  auto next_src = [&]() {
    const int32_t page = checked_page(ld_const(lc.bt_row + lc.pk), p.num_cache_blocks, bad_page);
    src = uniform64(page * page_bytes + (int64_t)lc.sub * kTile * row_stride);
  };
  auto advance_loader = [&]() {
    if (--lc_left > 0) {
      cursor_next<kTile>(lc, p, tpp);
      next_src();
    }
  };
  auto issue = [&](int stage) {
    DCP_LDS uint8_t* kdst = lds + stage * C::kStageBytes;
    DCP_LDS uint8_t* vdst = kdst + C::kHalfBytes;
#pragma unroll
    for (int k = 0; k < C::kCopies; ++k) {
      // head groups of a span read disjoint KV heads: every page byte has one reader
      copy16<true>(p.k_cache + src, ld_off[k], lds_addr(kdst + (k * KVW + wave) * 1024));
      copy16<true>(p.v_cache + src, ld_off[k], lds_addr(vdst + (k * KVW + wave) * 1024));
    }
  };

  // q[b, head, 32 s + 8 q4 .. +7]: the B operand of S^T = K Q^T for k-step s.  Lanes
  // of heads past the group load the group's first head: their columns are
  // independent of the others and never stored.  The loads are asm, so the
  // compiler's wait counting (which cannot see the copies either) does not drain
  // the ring before every use; the next request's slice goes to qnext ahead of a
  // copy round, and the loop's own wait covers it before it moves into qreg.
  // Column block c holds query token c of the pass (its slice QB * ... apart: the
  // tokens of a request are consecutive in q).
  bf16x8 qreg[QB][4], qnext[QB][4];
  // With four tokens the kernel needs more than 256 VGPRs and the compiler parks values
  // in accumulation registers: the slices are then ordinary loads, which the compiler
  // tracks (it waits for them, and for the copies issued after them, before their first
  // use, i.e. once per request), so no register can be moved before its load has landed.
  auto load_q = [&](bf16x8 (&dst)[QB][4], int b) {
#pragma unroll
    for (int c = 0; c < QB; ++c) {
      const uint16_t* qp = p.q + (int64_t)b * p.q_req_stride + ((int64_t)c * H + head) * kD + 8 * q4;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if constexpr (QB == 4)
          dst[c][s] = *(const bf16x8*)(qp + 32 * s);
        else
          asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "=v"(dst[c][s]) : "v"(qp), "n"(64 * s) : "memory");
      }
    }
  };
  auto settle = [&](bf16x8 (&r)[QB][4]) {
    if constexpr (QB != 4) {
#pragma unroll
      for (int c = 0; c < QB; ++c)
#pragma unroll
        for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(r[c][s]));
    }
  };

  f32x4 oacc[QB][8];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int c = 0; c < QB; ++c) {
#pragma unroll
    for (int m = 0; m < 8; ++m) oacc[c][m] = f32x4{};
    m_run[c] = -INFINITY;
    l_run[c] = 0.f;
  }

  // Finished pieces are stored after the next barrier, before that iteration's copies.
  // Query token c's row is H rows after token c - 1's, in the outputs and the pieces.
  bool pend = false;
  float pend_inv[QB], pend_lse[QB];
  float* pend_o = nullptr;  // token 0's row
  float* pend_l = nullptr;
  auto flush_piece = [&]() {
    if (pend) {
      if (head_ok) {
#pragma unroll
        for (int c = 0; c < QB; ++c) {
#pragma unroll
          for (int m = 0; m < 8; ++m)
            *(f32x4*)(pend_o + (int64_t)c * H * kD + 16 * m) = oacc[c][m] * pend_inv[c];
          if (q4 == 0) pend_l[c * H] = pend_lse[c];
        }
      }
#pragma unroll
      for (int c = 0; c < QB; ++c)
#pragma unroll
        for (int m = 0; m < 8; ++m) oacc[c][m] = f32x4{};
      pend = false;
    }
  };
  // Local tokens from which some column of the request may have to be masked: those
  // standing for the pass's QB - 1 newest positions (set per request).
  int mask_b = -1;
  int64_t mask_from = 0;

  // Zero the V rows nvalid..15 of the tile at `vb` (the V half of a stage).
  auto zero_tail = [&](DCP_LDS uint8_t* vb, int nvalid) {
    const int n = (kTile - nvalid) * C::kChunks;
    for (int e = tid; e < n; e += C::kThreads)
      zero_lds16(lds_addr(vb + nvalid * C::kRowBytes + e * 16));
  };

  // ---- prologue: query slice and the first kStages-1 tiles
  load_q(qreg, cc.b);
  // Compiler-tracked slices (QB = 4) must not reach the loop still pending: the wait
  // counting, blind to the asm copies issued after them, would otherwise keep a wait for
  // them in front of every tile's MFMAs, draining the copy ring each tile.
  if constexpr (QB == 4) wait_vmcnt_builtin<0>();
  next_src();
#pragma unroll
  for (int t = 0; t < C::kStages - 1; ++t) {
    issue(t);
    advance_loader();
  }
  int piece_t0 = cc.t;
  bool first_piece = true;
  bool q_moved = true;  // the slice for tile 0 was loaded before the prologue's copies

  for (int i = 0; i < total; ++i) {
    // Tile i has landed once only the copies of the kStages-2 younger tiles are
    // outstanding; after a query load (issued just before the previous copy round)
    // only that round may be, which also completes the load.  Piece stores sit
    // between copy rounds and only make the wait stricter.  The barrier then also
    // guarantees every wave has finished tile i-1, whose stage the copies below refill.
    if (q_moved) wait_vmcnt_builtin<C::kTileOps * (C::kStages - 2) - C::kTileOps * (C::kStages - 3)>();
    else wait_vmcnt_builtin<(C::kStages - 2) * C::kTileOps>();
    if (q_moved && i > 0) {
      settle(qnext);
#pragma unroll
      for (int c = 0; c < QB; ++c)
#pragma unroll
        for (int s = 0; s < 4; ++s) qreg[c][s] = qnext[c][s];
    }
    settle(qreg);
    q_moved = false;
    wg_barrier();
    wait_lgkm();
    flush_piece();
    const Cursor cur = cc;
    if (i + 1 < total) {
      cursor_next<kTile>(cc, p, tpp);
      if (cc.b != cur.b) {  // tile i+1 starts the next request: fetch its slice now
        load_q(qnext, cc.b);
        q_moved = true;
      }
    }
    issue((i + C::kStages - 1) % C::kStages);

    DCP_LDS uint8_t* kb = lds + (i % C::kStages) * C::kStageBytes;
    DCP_LDS uint8_t* vb = kb + C::kHalfBytes;
    const int nvalid = cur.Lr - cur.t * kTile;  // >= kTile for every tile but a request's last
    if (nvalid < kTile) {
      zero_tail(vb, nvalid);
      wait_lgkm();
      wg_barrier();
    }

    // ---- S^T [16 tokens x 16 heads] of each query token; a K operand serves all QB
    f32x4 sacc[QB];
#pragma unroll
    for (int c = 0; c < QB; ++c) sacc[c] = f32x4{};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 ka_s = *(const DCP_LDS bf16x8*)(kb + ka[s]);
#pragma unroll
      for (int c = 0; c < QB; ++c) sacc[c] = mfma16x16x32(ka_s, qreg[c][s], sacc[c]);
    }

    // ---- masks: rows past the request's end; with QB > 1, query token c sees the
    // global positions <= Lg - QB + c (Lg: the pass's length, its newest token's)
    float x[QB][4];
#pragma unroll
    for (int c = 0; c < QB; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[c][j] = 4 * q4 + j < nvalid ? sacc[c][j] * p.scale_log2 : -INFINITY;
    if constexpr (QB > 1) {
      const int N = p.part.num_ranks, I = p.part.interleave, r = p.part.rank;
      if (cur.b != mask_b) {
        mask_b = cur.b;
        mask_from = dcp_local_len((int64_t)cur.Lg - (QB - 1), N, I, r);
      }
      const int64_t j0 = (int64_t)cur.t * kTile;
      if (j0 + kTile > mask_from) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t g = dcp_global_index(j0 + 4 * q4 + j, N, I, r);
#pragma unroll
          for (int c = 0; c < QB; ++c)
            if (g > (int64_t)cur.Lg - QB + c) x[c][j] = -INFINITY;
        }
      }
    }

    // ---- online softmax (base 2) per query token; lane: head l16, tokens 4 q4 + j.  A
    // row that has seen no token yet keeps m = -inf with no NaN.
    bf16x4 pb[QB], pl[QB];  // P's high and low bf16 parts (see bf16_low_part)
    bool moved = false;
    bool big = false;  // some weight is more than kLowShare of its row's running sum
    float alpha[QB];
#pragma unroll
    for (int c = 0; c < QB; ++c) {
      float mloc = fmaxf(fmaxf(x[c][0], x[c][1]), fmaxf(x[c][2], x[c][3]));
      mloc = max_over_groups(mloc);
      const float m_new = mloc > m_run[c] + kRescaleSlack ? mloc : m_run[c];
      const bool none = m_new == -INFINITY;
      alpha[c] = none ? 1.f : fast_exp2(m_run[c] - m_new);
      float lsum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pr = none ? 0.f : fast_exp2(x[c][j] - m_new);
        lsum += pr;
        pb[c][j] = (__bf16)pr;
      }
      lsum = sum_over_groups(lsum);
      l_run[c] = l_run[c] * alpha[c] + lsum;
      moved = moved || m_new != m_run[c];
      m_run[c] = m_new;
      big = big || (!none && fast_exp2(mloc - m_new) > kLowShare * l_run[c]);
    }
    if (__any(moved)) {
#pragma unroll
      for (int c = 0; c < QB; ++c)
#pragma unroll
        for (int m = 0; m < 8; ++m) oacc[c][m] *= alpha[c];
    }

    // ---- O^T [128 dims x 16 heads] += V^T [128 x 16 tokens] P^T [16 x 16]; a V^T
    // operand serves all QB
    bf16x4 vam[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      vam[m] = __builtin_bit_cast(bf16x4, lds_read_tr16(vb + va[m]));
#pragma unroll
      for (int c = 0; c < QB; ++c) oacc[c][m] = mfma16x16x16(vam[m], pb[c], oacc[c][m]);
    }
    // with the low parts of the weights in a tile that needs them (see kLowShare)
    if (cur.Lr <= kLowAllTokens || __any(big)) {
#pragma unroll
      for (int c = 0; c < QB; ++c) {
        const bool none = m_run[c] == -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) pl[c][j] = bf16_low_part(none ? 0.f : fast_exp2(x[c][j] - m_run[c]), pb[c][j]);
#pragma unroll
        for (int m = 0; m < 8; ++m) oacc[c][m] = mfma16x16x16(vam[m], pl[c], oacc[c][m]);
      }
    }

    // ---- end of a request piece: normalisation and destination; stored after the
    // next barrier
    const bool last_of_req = cur.t == cur.ntile - 1;
    if (last_of_req || i == total - 1) {
      const bool whole = piece_t0 == 0 && last_of_req;
      const int64_t slot = 2 * w + (first_piece ? 0 : 1);
      pend = true;
#pragma unroll
      for (int c = 0; c < QB; ++c) {
        // a row that saw no token of the piece: O = 0, LSE = -inf
        pend_inv[c] = l_run[c] > 0.f ? 1.0f / l_run[c] : 0.f;
        pend_lse[c] = l_run[c] > 0.f ? (m_run[c] + fast_log2(l_run[c])) * kLn2 : -INFINITY;
        m_run[c] = -INFINITY;
        l_run[c] = 0.f;
      }
      pend_o = (whole ? p.out_o + ((int64_t)cur.b * p.out_req_rows + head) * kD : p.ws_o + (slot * rows + head) * kD) + 4 * q4;
      pend_l = whole ? p.out_lse + (int64_t)cur.b * p.out_req_rows + head : p.ws_lse + slot * rows + head;
      piece_t0 = 0;
      first_piece = false;
    }
    advance_loader();
  }
  flush_piece();
  if (bad_page && lane == 0) report_error(p.ws_err, kErrPageId);
  // No copy may still be landing in this work-group's LDS when it exits.
  wait_vmcnt_builtin<0>();
}

}  // namespace gqa

namespace {
template <int QB>
void launch_gqa_qb(const PartialParams& p, hipStream_t stream) {
  const int grid = p.part.num_parts * p.num_head_groups;
  switch (gqa_kv_heads_per_group(p.num_kv_heads)) {
    case 4: hipLaunchKernelGGL((gqa::gqa_partial_kernel<4, QB>), dim3(grid), dim3(256), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((gqa::gqa_partial_kernel<2, QB>), dim3(grid), dim3(128), 0, stream, p); break;
    default: hipLaunchKernelGGL((gqa::gqa_partial_kernel<1, QB>), dim3(grid), dim3(64), 0, stream, p); break;
  }
}
}  // namespace

hipError_t launch_gqa_partial(const PartialParams& p, hipStream_t stream) {
  switch (p.q_block) {
    case 1: launch_gqa_qb<1>(p, stream); break;
    case 2: launch_gqa_qb<2>(p, stream); break;
    case 4: launch_gqa_qb<4>(p, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dcp
