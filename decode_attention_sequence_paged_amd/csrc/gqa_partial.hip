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

template <int KVW>
__global__ __launch_bounds__(64 * KVW, 1) void gqa_partial_kernel(PartialParams p) {
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
  bf16x8 qreg[4], qnext[4];
  auto load_q = [&](bf16x8 (&dst)[4], int b) {
    const uint16_t* qp = p.q + (int64_t)b * p.q_req_stride + (int64_t)head * kD + 8 * q4;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "=v"(dst[s]) : "v"(qp), "n"(64 * s) : "memory");
  };
  auto settle = [&](bf16x8 (&r)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(r[s]));
  };

  f32x4 oacc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) oacc[m] = f32x4{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  // Finished pieces are stored after the next barrier, before that iteration's copies.
  bool pend = false;
  float pend_inv = 0.f, pend_lse = 0.f;
  float* pend_o = nullptr;
  float* pend_l = nullptr;
  auto flush_piece = [&]() {
    if (pend) {
      if (head_ok) {
#pragma unroll
        for (int m = 0; m < 8; ++m) *(f32x4*)(pend_o + 16 * m) = oacc[m] * pend_inv;
        if (q4 == 0) *pend_l = pend_lse;
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) oacc[m] = f32x4{};
      pend = false;
    }
  };

  // Zero the V rows nvalid..15 of the tile at `vb` (the V half of a stage).
  auto zero_tail = [&](DCP_LDS uint8_t* vb, int nvalid) {
    const int n = (kTile - nvalid) * C::kChunks;
    for (int e = tid; e < n; e += C::kThreads)
      zero_lds16(lds_addr(vb + nvalid * C::kRowBytes + e * 16));
  };

  // ---- prologue: query slice and the first kStages-1 tiles
  load_q(qreg, cc.b);
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
      for (int s = 0; s < 4; ++s) qreg[s] = qnext[s];
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

    // ---- S^T [16 tokens x 16 heads]
    f32x4 sacc = f32x4{};
#pragma unroll
    for (int s = 0; s < 4; ++s) sacc = mfma16x16x32(*(const DCP_LDS bf16x8*)(kb + ka[s]), qreg[s], sacc);

    // ---- online softmax (base 2); lane: head l16, tokens 4 q4 + j
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = 4 * q4 + j < nvalid ? sacc[j] * p.scale_log2 : -INFINITY;
    float mloc = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mloc = max_over_groups(mloc);
    const float m_new = mloc > m_run + kRescaleSlack ? mloc : m_run;
    const float alpha = fast_exp2(m_run - m_new);
    float lsum = 0.f;
    bf16x4 pb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pr = fast_exp2(x[j] - m_new);
      lsum += pr;
      pb[j] = (__bf16)pr;
    }
    lsum = sum_over_groups(lsum);
    l_run = l_run * alpha + lsum;
    if (__any(m_new != m_run)) {
#pragma unroll
      for (int m = 0; m < 8; ++m) oacc[m] *= alpha;
    }
    m_run = m_new;

    // ---- O^T [128 dims x 16 heads] += V^T [128 x 16 tokens] P^T [16 x 16]
#pragma unroll
    for (int m = 0; m < 8; ++m)
      oacc[m] = mfma16x16x16(__builtin_bit_cast(bf16x4, lds_read_tr16(vb + va[m])), pb, oacc[m]);

    // ---- end of a request piece: normalisation and destination; stored after the
    // next barrier
    const bool last_of_req = cur.t == cur.ntile - 1;
    if (last_of_req || i == total - 1) {
      const bool whole = piece_t0 == 0 && last_of_req;
      const int64_t slot = 2 * w + (first_piece ? 0 : 1);
      pend = true;
      // a row that saw no token of the piece: O = 0, LSE = -inf
      pend_inv = l_run > 0.f ? 1.0f / l_run : 0.f;
      pend_lse = l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : -INFINITY;
      pend_o = (whole ? p.out_o + ((int64_t)cur.b * p.out_req_rows + head) * kD : p.ws_o + (slot * H + head) * kD) + 4 * q4;
      pend_l = whole ? p.out_lse + (int64_t)cur.b * p.out_req_rows + head : p.ws_lse + slot * H + head;
      piece_t0 = 0;
      first_piece = false;
      m_run = -INFINITY;
      l_run = 0.f;
    }
    advance_loader();
  }
  flush_piece();
  if (bad_page && lane == 0) report_error(p.ws_err, kErrPageId);
  // No copy may still be landing in this work-group's LDS when it exits.
  wait_vmcnt_builtin<0>();
}

}  // namespace gqa

hipError_t launch_gqa_partial(const PartialParams& p, hipStream_t stream) {
  const int grid = p.part.num_parts * p.num_head_groups;
  switch (gqa_kv_heads_per_group(p.num_kv_heads)) {
    case 4: hipLaunchKernelGGL(gqa::gqa_partial_kernel<4>, dim3(grid), dim3(256), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(gqa::gqa_partial_kernel<2>, dim3(grid), dim3(128), 0, stream, p); break;
    default: hipLaunchKernelGGL(gqa::gqa_partial_kernel<1>, dim3(grid), dim3(64), 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace dcp
