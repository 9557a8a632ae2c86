// MLA partial decode attention over one rank's shard of a paged latent KV cache.
//
// What it computes (vLLM blog "Efficient Decode Context Parallelism with vLLM for
// Long Context Workloads", Sec. 4.1 "Compute" and Sec. 5.3 "MLA Backend"): every
// query head attends the rank's local latent rows; K is the whole 576-dim row and
// V its first 512 entries (the weight-absorbed form, where the query is already in
// the latent space).  Output: normalised partial O [B,H,512] and LSE [B,H].
//
// Design for gfx950:
//  * A work-group owns up to 64 query heads and a token-balanced span of the rank's
//    32-token tiles; the span may cover the end of one request, whole requests and
//    the start of another.  Every latent row is read from HBM once per head group
//    and serves as both K and V.
//  * Tiles stream HBM -> LDS through a 4-stage ring of 16-byte direct-to-LDS copies
//    (no VGPR staging).  A tile is 32 rows of 72 16-byte slots; inside each row the
//    chunks are XOR-swizzled in groups of 8, which makes both operand read patterns
//    free of LDS bank conflicts while a tile stays exactly 36 copy instructions.
//  * The work-group is a grid of waves: head halves (32 heads each) x partners.  The
//    two partners of a head half split the 576 score dims (even / odd 32-dim
//    steps): each computes partial scores of its 32 heads against all 32 tokens of
//    the tile (S^T = K Q^T, 16x16x32 bf16 MFMA, tokens on the rows; one K operand
//    read feeds both 16-head blocks) and hands the partial of the other's head block
//    over through LDS.  Each wave then owns 16 heads: it adds the two partials, runs
//    the base-2 online softmax over the 32 tokens and accumulates O^T += V^T P^T for
//    its heads over all 512 dims, V^T coming from LDS through the transposing
//    ds_read_b64_tr_b16.  K is read from LDS by two waves rather than by every wave,
//    and no softmax is evaluated twice.  The wave's 32 x 288 query slice and its
//    16 x 512 O accumulator live in accumulation registers (AGPR-form MFMA), which
//    leaves the VGPRs to deep operand prefetch.
//  * The copies of tile i+3 are spread between the P.V MFMAs of tile i, so their
//    issue (which stalls while the memory pipeline is full) hides under the matrix
//    pipe.  Copy issue has no branches: past the end of the span the last tile is
//    copied again into a stage nobody reads.
//  * Rows of a request's last, partial tile past its end are copied from the page
//    like any other row (they stay inside the page) and are made inert: their scores
//    are set to -inf and their V part is zeroed in LDS before it is read.
//  * The running maximum moves only when a tile's maximum exceeds it by more than
//    kRescaleSlack (log2 units), so the 128-register O accumulator is rarely
//    rescaled; P stays <= 2^kRescaleSlack and the final LSE uses the same maximum,
//    so the result is unchanged.
//  * P enters the P.V MFMAs as its bf16 high part and, in the tiles where a weight is
//    a sizeable share of its row, also as its bf16 low part (bf16_low_part in
//    dcp_device.h), so that short requests keep about 16 bits of every weight.
#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {
namespace mla {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;            // 1152
constexpr int kChunks = kRowBytes / 16;        // 72 16-byte chunks per row
constexpr int kTile = 32;                      // tokens per tile
constexpr int kTileBytes = kTile * kRowBytes;  // 36864: LDS tile = global tile
constexpr int kCopyInstr = kTileBytes / 1024;  // 36 wave-wide 16-byte copies per tile
constexpr int kStages = 4;
constexpr int kKSteps = kDqk / 32;             // 18 k-steps of 32 dims
constexpr int kKStepsWave = kKSteps / 2;       // 9 per partner (even / odd steps)
constexpr int kVBlocks = kDv / 16;             // 32 O^T blocks of 16 dims
constexpr int kPrefetchK = 3;                  // K operand steps (2 reads each) issued ahead
constexpr int kPrefetchV = 8;                  // V^T operand steps (2 reads each) issued ahead
constexpr float kRescaleSlack = 8.0f;
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// XOR swizzle of the chunks of tile row r inside their aligned group of 8.  With a
// row stride of 72 slots (8 mod 16), the 16-byte bank group of (r, c) is
// 8*(r%2) + (c ^ x(r)) mod 16.  gfx950 serves a ds_read_b128 in four passes of 16
// lanes: within each half of the wave, the lane quads (lane / 4) of even popcount
// form one pass and those of odd popcount the other (measured).  The K operand read
// puts lane (q4, l16) on row l16 and chunk 4 s + q4 of one 32-dim step;
// x(r) = r & 6 gives the 16 lanes of every pass 16 distinct bank groups, and it
// keeps the transposed V read (64 lanes x 8 bytes: rows 4 q4 + l16/4, one even/odd
// chunk pair) at two lanes per bank, which that read serves without conflict.
__device__ __forceinline__ constexpr int row_swz(int r) { return r & 6; }

// NH head halves of 32 heads per work-group; 2 * NH waves (head halves x partners).
template <int NH>
struct Cfg {
  static constexpr int kWaves = 2 * NH;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kHeads = 32 * NH;
  static constexpr int kCopies = kCopyInstr / kWaves;  // copy instructions per wave per tile
  static_assert(kCopyInstr % kWaves == 0, "copies must split evenly over waves");
  static_assert(2 * kCopies < 64, "vmcnt range");
};

// Exchange of partial scores through LDS.  Written as asm: the compiler's wait
// counting cannot tell the exchange buffer from the stages the in-flight
// direct-to-LDS copies write, and would drain those copies before every access.
// The read waits for its own data; the writes are completed by the caller's wait
// before the barrier.  Two 16-byte slots, 1024 bytes apart (token blocks 0 and 1).
__device__ __forceinline__ void read_scores(uint32_t addr, f32x4& a, f32x4& b) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %2 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(a), "=v"(b)
      : "v"(addr)
      : "memory");
}
__device__ __forceinline__ void write_scores(uint32_t addr, f32x4 a, f32x4 b) {
  asm volatile(
      "ds_write_b128 %0, %1\n\t"
      "ds_write_b128 %0, %2 offset:1024"
      :
      : "v"(addr), "v"(a), "v"(b)
      : "memory");
}
template <int NH>
__global__ __launch_bounds__(128 * NH, 1) void mla_partial_kernel(PartialParams p) {
  using C = Cfg<NH>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kTileBytes];
  __shared__ __attribute__((aligned(16))) f32x4 s_xch[NH * 2 * 2 * 64];  // [hh][writer kk][token block][lane]
  __shared__ int64_t s_scan[C::kThreads];
  __shared__ int64_t s_loc[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int kk = wave & 1;          // score dims of k-steps 2 s + kk; head block of its softmax and O
  const int hh = wave >> 1;         // head half
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  int64_t w;
  int hg;
  block_to_span(p.part.num_parts, p.num_head_groups, &w, &hg);
  const bool write_prefix = (w == 0 && hg == 0);
  const SpanLoc loc = locate_span<C::kThreads>(p.part, w, write_prefix ? p.ws_prefix : nullptr,
                                               p.ws_err, s_scan, s_loc);
  if (loc.start >= loc.end) return;
  const int total = (int)(loc.end - loc.start);
  const int tpp = p.block_size / kTile;                    // tiles per page
  const int64_t page_bytes = (int64_t)p.block_size * kRowBytes;

  const int H = p.num_q_heads;
  const int head0 = hg * C::kHeads + hh * 32 + l16;  // this lane's score column in head block 0 (+16: 1)
  const int head = head0 + 16 * kk;                  // this lane's head for softmax and O
  DCP_LDS uint8_t* lds = (DCP_LDS uint8_t*)smem;

  // This lane's copies: LDS slot s = (k * kWaves + wave) * 64 + lane of a tile is
  // position s % 72 of row s / 72, which holds chunk (pos ^ row_swz(row)).
  uint32_t ld_off[C::kCopies];
#pragma unroll
  for (int k = 0; k < C::kCopies; ++k) {
    const int s = (k * C::kWaves + wave) * 64 + lane;
    const int row = s / kChunks;
    const int pos = s - row * kChunks;
    ld_off[k] = (uint32_t)(row * kRowBytes + (pos ^ row_swz(row)) * 16);
  }

  // Operand read offsets inside a stage.  K: token block tb, row 16 tb + l16, chunk
  // 4 s + q4 of k-step s = 2 s' + kk -> kb[tb] + 128 s'.  V: row 4 q4 + l16 / 4 (+16
  // rows for the second token block), dims 16 m + 4 (l16 % 4) .. +3, i.e. chunk
  // 2 m + (l16 % 4) / 2, byte half l16 % 2 -> vb[m & 3] + 128 (m >> 2).
  uint32_t kb[2], vb[4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int r = 16 * tb + l16;
    const int x = row_swz(r);
    kb[tb] = (uint32_t)(r * kRowBytes + 64 * (kk ^ (x >> 2)) + 16 * (q4 ^ (x & 3)));
  }
  {
    const int r = 4 * q4 + (l16 >> 2);
    const int x = row_swz(r);
    const int h = (l16 & 3) >> 1;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      vb[v] = (uint32_t)(r * kRowBytes + 32 * (v ^ (x >> 1)) + 16 * (h ^ (x & 1)) + 8 * (l16 & 1));
  }

  Cursor lc, cc;
  cursor_set(lc, p, tpp, loc.b0, (int)loc.off0);
  cc = lc;

  // Copy source: the tile the loader cursor is on.  Past the end of the span the
  // cursor stays on the last tile, which is then copied again (into a stage no wave
  // reads) so that the copy code in the loop needs no branch.
  int lc_left = total;  // tiles the loader has not moved past yet
  const uint8_t* src = nullptr;
  bool bad_page = false;
  auto next_src = [&]() {
    const int32_t page = checked_page(ld_const(lc.bt_row + lc.pk), p.num_cache_blocks, bad_page);
    src = p.k_cache + page * page_bytes + lc.sub * kTileBytes;
  };
  auto advance_loader = [&]() {
    if (--lc_left > 0) {
      cursor_next(lc, p, tpp);
      next_src();
    }
  };
  auto issue_copy = [&](int k, int stage) {
    copy16<true>(src, ld_off[k], lds_addr(lds + stage * kTileBytes + (k * C::kWaves + wave) * 1024));
  };

  // q[b, head0 + 16 hb, 32 (2 s' + kk) + 8 q4 .. +7]: the B operand of S^T = K Q^T
  // for head block hb and this wave's k-step s'.  It is only an MFMA operand, so it
  // is loaded straight into accumulation registers.  Lanes of heads past H load
  // head 0's slice: their score columns are independent of the others and never
  // stored.  The loads are not tracked by the compiler's wait counting; the loop's
  // explicit vmcnt waits cover them (memory clobber: they stay in program order
  // with the tile copies).
  bf16x8 qreg[2][kKStepsWave];
  auto load_q = [&](int b) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int hd = head0 + 16 * hb;
      const uint16_t* qp = p.q + ((int64_t)b * H + (hd < H ? hd : 0)) * kDqk + 32 * kk + 8 * q4;
#pragma unroll
      for (int s = 0; s < kKStepsWave; ++s)
        asm volatile("global_load_dwordx4 %0, %1, off offset:%2"
                     : "=a"(qreg[hb][s]) : "v"(qp), "n"(128 * s) : "memory");
    }
  };

  // Partial S^T [32 tokens x 32 heads] over this wave's 9 k-steps of the tile at
  // `tb`: four accumulation chains (token block x head block); one K read feeds
  // both head blocks.
  auto qk = [&](const DCP_LDS uint8_t* tb, f32x4 (&sacc)[2][2]) {
#pragma unroll
    for (int a = 0; a < 2; ++a) sacc[a][0] = sacc[a][1] = f32x4{};
    bf16x8 r[kPrefetchK][2];
#pragma unroll
    for (int s = 0; s < kPrefetchK; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) r[s][t] = *(const DCP_LDS bf16x8*)(tb + kb[t] + 128 * s);
#pragma unroll
    for (int s = 0; s < kKStepsWave; ++s) {
      bf16x8 a[2] = {r[s % kPrefetchK][0], r[s % kPrefetchK][1]};
      const int sn = s + kPrefetchK;
      if (sn < kKStepsWave) {
#pragma unroll
        for (int t = 0; t < 2; ++t) r[s % kPrefetchK][t] = *(const DCP_LDS bf16x8*)(tb + kb[t] + 128 * sn);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sacc[t][0] = mfma16x16x32(a[t], qreg[0][s], sacc[t][0]);
        sacc[t][1] = mfma16x16x32(a[t], qreg[1][s], sacc[t][1]);
      }
    }
    // Keep kPrefetchK steps of operand reads in flight: reads first, then
    // (4 MFMA, 2 reads) ...
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPrefetchK, 0);
#pragma unroll
    for (int s = 0; s < kKStepsWave - kPrefetchK; ++s) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4 * kPrefetchK, 0);
  };

  // Running softmax state of this lane's head: maximum (log2 units), sum, and P^T
  // of the tile as the B operand of its P.V.
  float m_run = -INFINITY;
  float l_run = 0.f;
  CausalFrom cfrom;
  bf16x8 pb, pl;  // P's high and low bf16 parts (see bf16_low_part)
  float alpha = 1.f;
  bool moved = false;
  bool need_lo = false;  // the tile takes the low parts (see kLowShare)
  // Softmax over the tile's 32 scores of this lane's head (x[0..3]: tokens 4 q4 + j,
  // x[4..7]: tokens 16 + 4 q4 + j).
  auto softmax = [&](const f32x4& s0, const f32x4& s1, bool all_lo) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) { x[j] = s0[j]; x[j + 4] = s1[j]; }
    float mloc = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                       fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mloc = max_over_groups(mloc);
    const float m_new = mloc > m_run + kRescaleSlack ? mloc : m_run;
    // no visible token yet (a causally masked row): nothing to weigh or rescale
    const bool none = m_new == -INFINITY;
    alpha = none ? 1.f : fast_exp2(m_run - m_new);
    moved = m_new != m_run;
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float pr = none ? 0.f : fast_exp2(x[j] - m_new);
      lsum += pr;
      pb[j] = (__bf16)pr;
    }
    lsum = sum_over_groups(lsum);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    // mloc is the row's maximum over the tile
    need_lo = all_lo || __any(!none && fast_exp2(mloc - m_new) > kLowShare * l_run);
    if (need_lo) {
#pragma unroll
      for (int j = 0; j < 8; ++j) pl[j] = bf16_low_part(none ? 0.f : fast_exp2(x[j] - m_new), pb[j]);
    }
  };

  f32x4 oacc[kVBlocks];
#pragma unroll
  for (int m = 0; m < kVBlocks; ++m) oacc[m] = f32x4{};

  // O^T [512 dims x 16 heads] += V^T [512 x 32 tokens] P^T [32 x 16] for the tile at
  // `tb`, with this wave's copies of a later tile (into `stage`) spread between the
  // MFMAs: the copy asm orders itself with the LDS reads around it, so its place in
  // the source is its place in the instruction stream.  Source lane l16 of each
  // 16-lane group addresses row 4 q4 + l16 / 4 (and +16); lane i then holds dim
  // 16 m + i of the tokens P's element j stands for.
  auto pv = [&](const DCP_LDS uint8_t* tb, int stage, auto lo_tag) {
    constexpr bool kLo = decltype(lo_tag)::value;
    u32x2 v1[kPrefetchV], v2[kPrefetchV];
#pragma unroll
    for (int m = 0; m < kPrefetchV; ++m) {
      v1[m] = lds_read_tr16(tb + vb[m & 3] + 128 * (m >> 2));
      v2[m] = lds_read_tr16(tb + vb[m & 3] + 128 * (m >> 2) + 16 * kRowBytes);
    }
#pragma unroll
    for (int m = 0; m < kVBlocks; ++m) {
      const bf16x8 a = join_tr16(v1[m % kPrefetchV], v2[m % kPrefetchV]);
      const int mn = m + kPrefetchV;
      if (mn < kVBlocks) {
        v1[m % kPrefetchV] = lds_read_tr16(tb + vb[mn & 3] + 128 * (mn >> 2));
        v2[m % kPrefetchV] = lds_read_tr16(tb + vb[mn & 3] + 128 * (mn >> 2) + 16 * kRowBytes);
      }
#pragma unroll
      for (int k = 0; k < C::kCopies; ++k)
        if (k * kVBlocks / C::kCopies == m) issue_copy(k, stage);
      oacc[m] = mfma16x16x32(a, pb, oacc[m]);
      if constexpr (kLo) oacc[m] = mfma16x16x32(a, pl, oacc[m]);
    }
  };

  // Zero the V part (chunks 0..63 = positions 0..63: the swizzle keeps groups of 8)
  // of rows nvalid..31 of the tile at `tb`.
  auto zero_tail = [&](const DCP_LDS uint8_t* tb, int nvalid) {
    const int n = (kTile - nvalid) * 64;
    for (int e = tid; e < n; e += C::kThreads)
      zero_lds16(lds_addr(tb + (nvalid + (e >> 6)) * kRowBytes + (e & 63) * 16));
  };

  // Exchange slots: this wave writes the partial of the partner's head block, reads
  // the partner's partial of its own.
  const uint32_t xch_out = lds_addr((const DCP_LDS f32x4*)s_xch + (hh * 4 + kk * 2) * 64 + lane);
  const uint32_t xch_in = lds_addr((const DCP_LDS f32x4*)s_xch + (hh * 4 + (kk ^ 1) * 2) * 64 + lane);

  // ---- prologue: query slice, then three tiles in flight
  load_q(cc.b);
  next_src();
  for (int s = 0; s < kStages - 1; ++s) {
#pragma unroll
    for (int k = 0; k < C::kCopies; ++k) issue_copy(k, s);
    advance_loader();
  }
  int issued = kStages - 1;  // copy rounds issued (the last ones may repeat a tile)
  int q_after = 0;           // copy rounds issued before the newest query load
  int piece_t0 = cc.t;       // first tile of the current piece inside request cc.b
  bool first_piece = true;

  // A finished piece is stored at the top of the next iteration, right after its
  // barrier and before that iteration's copies.  Stored at once, its stores would be
  // the youngest memory operations at the next tile wait, which could then only be
  // met by draining every copy in flight; deferred, they sit between two copy
  // rounds, and the wait completes them together with the older round.
  bool pend = false;
  float pend_inv = 0.f, pend_lse = 0.f;
  float* pend_o = nullptr;
  float* pend_l = nullptr;
  auto flush_piece = [&]() {
    if (pend) {
      if (head < H) {
#pragma unroll
        for (int m = 0; m < kVBlocks; ++m) *(f32x4*)(pend_o + 16 * m) = oacc[m] * pend_inv;
        if (q4 == 0) *pend_l = pend_lse;
      }
#pragma unroll
      for (int m = 0; m < kVBlocks; ++m) oacc[m] = f32x4{};
      pend = false;
    }
  };

  for (int i = 0; i < total; ++i) {
    // Tile i (and the newest query slice) have landed once only the copy rounds
    // issued after both are outstanding; younger memory operations only make the
    // wait stricter.  The barrier then also guarantees every wave has finished the
    // P.V of tile i-1, whose stage this iteration's copies refill.
    {
      const int after_tile = issued - (i + 1);
      const int after_q = issued - q_after;
      const int after = after_tile < after_q ? after_tile : after_q;
      if (after >= 2) wait_vmcnt_builtin<2 * C::kCopies>();
      else if (after == 1) wait_vmcnt_builtin<C::kCopies>();
      else wait_vmcnt_builtin<0>();
    }
    wg_barrier();
    // The loader's scalar loads were issued an iteration ago; retiring them here
    // lets the operand reads below wait for single LDS accesses, not for lgkmcnt(0).
    wait_lgkm();
    flush_piece();
    const DCP_LDS uint8_t* tb = lds + (i % kStages) * kTileBytes;
    const Cursor cur = cc;
    const int nvalid = cur.Lr - cur.t * kTile;  // >= kTile for every tile but a request's last
    if (nvalid < kTile) zero_tail(tb, nvalid);

    f32x4 sacc[2][2];
    qk(tb, sacc);
    // The next request's query slice as soon as this one's last scores are done,
    // ahead of the copies issued below.
    if (i + 1 < total) {
      cursor_next(cc, p, tpp);
      if (cc.b != cur.b) {
        load_q(cc.b);
        q_after = issued;
      }
    }
    write_scores(xch_out, kk ? sacc[0][0] : sacc[0][1], kk ? sacc[1][0] : sacc[1][1]);
    wait_lgkm();
    wg_barrier();
    f32x4 s0, s1;
    read_scores(xch_in, s0, s1);
    s0 = ((kk ? sacc[0][1] : sacc[0][0]) + s0) * p.scale_log2;
    s1 = ((kk ? sacc[1][1] : sacc[1][0]) + s1) * p.scale_log2;
    if (nvalid < kTile) {
      // tokens past the end: rows 4 q4 + j (block 0) and 16 + 4 q4 + j (block 1)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (4 * q4 + j >= nvalid) s0[j] = -INFINITY;
        if (16 + 4 * q4 + j >= nvalid) s1[j] = -INFINITY;
      }
    }
    causal_mask(p, cur, nvalid, head, q4, s0, s1, cfrom);
    softmax(s0, s1, cur.Lr <= kLowAllTokens);
    if (__any(moved)) {
#pragma unroll
      for (int m = 0; m < kVBlocks; ++m) oacc[m] *= alpha;
    }
    if (need_lo) pv(tb, issued % kStages, std::true_type{});
    else pv(tb, issued % kStages, std::false_type{});
    ++issued;

    // ---- end of a request piece: its normalisation and destination; the stores
    // follow after the next barrier
    const bool last_of_req = cur.t == cur.ntile - 1;
    if (last_of_req || i == total - 1) {
      const bool whole = piece_t0 == 0 && last_of_req;
      const int64_t slot = 2 * w + (first_piece ? 0 : 1);
      pend = true;
      // a row that saw no token of the piece: O = 0, LSE = -inf
      pend_inv = l_run > 0.f ? 1.0f / l_run : 0.f;
      pend_lse = l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : -INFINITY;
      const int hd = head < H ? head : 0;
      pend_o = (whole ? p.out_o + ((int64_t)cur.b * H + hd) * kDv : p.ws_o + (slot * H + hd) * kDv) + 4 * q4;
      pend_l = whole ? p.out_lse + (int64_t)cur.b * H + hd : p.ws_lse + slot * H + hd;
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


// ------------------------------------------------------------------ 64-head groups
// A work-group of 12 waves (three per SIMD) in two roles, one tile apart:
//  * score waves 0..3: wave s owns head block s (16 heads) and all 576 score dims.
//    It computes S^T of tile j+1 (16x16x32 MFMA, four accumulation chains: token
//    block x k-step parity), runs the online softmax and leaves P^T (bf16, laid out
//    as the MFMA B operand), the rescale factor of each head and, at the end of a
//    piece, 1/l in LDS; it stores the piece's LSE itself.  In a tile where its head
//    block needs them it also leaves the low parts of P (fp8-coded) and a flag.
//  * P.V waves 4..11: wave v owns output dims 64 v .. 64 v + 63 of all 64 heads
//    (16 O^T accumulators of 16 dims x 16 heads).  During tile j's interval it
//    rescales, accumulates O^T += V^T P^T for tile j (a second pass adds the low
//    parts of the head blocks that left them) and stores finished pieces;
//    the first four also issue the copies of tile j+3 into the stage tile j-1 has
//    just released.
// Each role therefore keeps the matrix pipe busy while the other waits on a
// latency-bound step (the softmax, the copies), and the two meet once per tile at a
// single barrier.  V^T is read from LDS once per tile (each P.V wave reads only
// its own dims) and K four times (once per head block).  Splitting the P.V work
// over eight waves instead of four puts a third wave on every SIMD: multi-query
// calls, whose per-tile work is compute- and latency-bound, gain about 5%, and the
// single-query calls, bound by HBM, are unchanged.
namespace wide {
constexpr int kRoleWaves = 4;                   // score waves (one per SIMD)
constexpr int kCopyWaves = 4;                   // P.V waves that issue the tile copies
constexpr int kCopies = kCopyInstr / kCopyWaves;  // 9 copy instructions per copying wave and tile
constexpr int kHeadBlocks = 4;
constexpr int kPfK = 4;                         // K operand steps in flight (2 reads each)
constexpr int kPfV = 4;                         // V^T operand blocks in flight (2 reads each)
constexpr int kPVWaves = 8;                     // the P.V wave count launched
static_assert(kCopyInstr % kCopyWaves == 0, "copies must split evenly over the copying waves");
// kPV P.V waves (4 or 8), each owning kDv / kPV output dims of the 64 heads.
template <int kPV>
struct PV {
  static constexpr int kThreads = 64 * (kRoleWaves + kPV);
  static constexpr int kDims = kDv / kPV;               // output dims per P.V wave
  static constexpr int kDimBlocks = kDims / 16;         // O^T dim blocks per P.V wave
  static constexpr int kChunksPerRow = kDims * 2 / 16;  // its 16-byte chunks of a row's V part
  static_assert(kPV == 4 || kPV == 8, "P.V waves");
};
}  // namespace wide

// kStream: one head group (every page has one reader), see copy16.  kPV: P.V waves.
template <bool kStream, int kPV>
__global__ __launch_bounds__(wide::PV<kPV>::kThreads, 1) void mla_partial_wide_kernel(PartialParams p) {
  using namespace wide;
  using PVC = PV<kPV>;
  constexpr int kThreads = PVC::kThreads;
  constexpr int kDimBlocks = PVC::kDimBlocks;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kTileBytes];
  __shared__ __attribute__((aligned(16))) bf16x8 s_p[2][kHeadBlocks][64];  // [tile parity][head block][lane]
  __shared__ __attribute__((aligned(16))) u32x2 s_pl[2][kHeadBlocks][64];   // the low parts, fp8-coded
  __shared__ __attribute__((aligned(16))) float s_alpha[2][16][kHeadBlocks];  // [parity][head in block][block]
  __shared__ __attribute__((aligned(16))) float s_inv[2][16][kHeadBlocks];
  __shared__ __attribute__((aligned(16))) int s_lo[2][16][kHeadBlocks];  // the head block's tile took the low parts
  __shared__ int64_t s_loc[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  int64_t w;
  int hg;
  block_to_span(p.part.num_parts, p.num_head_groups, &w, &hg);
  const bool write_prefix = (w == 0 && hg == 0);
  // The span scan's scratch lives in the first stage, before any copy lands there.
  const SpanLoc loc = locate_span<kThreads>(p.part, w, write_prefix ? p.ws_prefix : nullptr,
                                            p.ws_err, (int64_t*)smem, s_loc);
  if (loc.start >= loc.end) return;
  const int total = (int)(loc.end - loc.start);
  const int tpp = p.block_size / kTile;
  const int64_t page_bytes = (int64_t)p.block_size * kRowBytes;
  const int H = p.num_q_heads;
  const int hbase = hg * 64;
  DCP_LDS uint8_t* lds = (DCP_LDS uint8_t*)smem;

  Cursor cur0;
  cursor_set(cur0, p, tpp, loc.b0, (int)loc.off0);

  // Where a piece ending at `cur` goes: the request's final row if the span holds
  // the whole request, else the span's first or last workspace slot.
  struct Piece {
    int t0;
    bool first;
  };
  auto piece_row = [&](const Piece& pc, const Cursor& cur, int head, bool& whole) -> int64_t {
    whole = pc.t0 == 0 && cur.t == cur.ntile - 1;
    const int64_t slot = 2 * w + (pc.first ? 0 : 1);
    return whole ? (int64_t)cur.b * H + head : slot * H + head;
  };

  if (wave < kRoleWaves) {
    // ================================================================ score waves
    const int sb = wave;                       // head block
    const int head = hbase + 16 * sb + l16;   // this lane's score column
    const bool head_ok = head < H;

    // K operand of token block tb, k-step s: row 16 tb + l16, chunk 4 s + q4
    // -> kb[tb][s & 1] + 128 (s >> 1) under the row swizzle.
    uint32_t kb[2][2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int r = 16 * tb + l16;
      const int x = row_swz(r);
#pragma unroll
      for (int par = 0; par < 2; ++par)
        kb[tb][par] = (uint32_t)(r * kRowBytes + 64 * (par ^ (x >> 2)) + 16 * (q4 ^ (x & 3)));
    }

    // q[b, head, 32 s + 8 q4 .. +7] for the 18 k-steps: the B operand of S^T = K Q^T.
    // Not tracked by the compiler's wait counting: the explicit vmcnt wait before the
    // barrier that precedes its first use covers it.
    bf16x8 qreg[kKSteps];
    auto load_q = [&](int b) {
      const uint16_t* qp = p.q + ((int64_t)b * H + (head_ok ? head : 0)) * kDqk + 8 * q4;
#pragma unroll
      for (int s = 0; s < kKSteps; ++s)
        asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "=v"(qreg[s]) : "v"(qp), "n"(64 * s) : "memory");
    };

    auto qk = [&](const DCP_LDS uint8_t* tb, f32x4& s0, f32x4& s1) {
      f32x4 acc[2][2];
#pragma unroll
      for (int a = 0; a < 2; ++a) acc[a][0] = acc[a][1] = f32x4{};
      bf16x8 r[kPfK][2];
#pragma unroll
      for (int s = 0; s < kPfK; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t) r[s][t] = *(const DCP_LDS bf16x8*)(tb + kb[t][s & 1] + 128 * (s >> 1));
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) {
        const bf16x8 a0 = r[s % kPfK][0], a1 = r[s % kPfK][1];
        const int sn = s + kPfK;
        if (sn < kKSteps) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
            r[s % kPfK][t] = *(const DCP_LDS bf16x8*)(tb + kb[t][sn & 1] + 128 * (sn >> 1));
        }
        acc[0][s & 1] = mfma16x16x32(a0, qreg[s], acc[0][s & 1]);
        acc[1][s & 1] = mfma16x16x32(a1, qreg[s], acc[1][s & 1]);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPfK, 0);
#pragma unroll
      for (int s = 0; s < kKSteps - kPfK; ++s) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * kPfK, 0);
      s0 = acc[0][0] + acc[0][1];
      s1 = acc[1][0] + acc[1][1];
    };

    float m_run = -INFINITY, l_run = 0.f;
    CausalFrom cfrom;
    Cursor sc = cur0;
    Piece pc{sc.t, true};
    bool q_pending = true;
    load_q(sc.b);
    wait_vmcnt_builtin<0>();
    q_pending = false;
    wg_barrier();  // tile 0 has landed

    for (int j = 0; j < total; ++j) {
      const Cursor cur = sc;
      const int par = j & 1;
      const DCP_LDS uint8_t* tb = lds + (j % kStages) * kTileBytes;
      // The head block's tile takes the low parts of its weights (see kLowShare) if one
      // of them is above kLowShare of the row sum after the tile.  That sum is at least
      // the sum before the tile (rescaled) plus the weight itself, so a weight P of it
      // qualifies if P (1 - kLowShare) > kLowShare l_prev alpha, which flags every tile
      // that needs it: in log2 units against the running maximum, log2 P > lo_thr.  The
      // threshold's cross-lane adds and logarithm overlap the score MFMAs.
      float lo_thr = fast_log2(kLowShare / (1.f - kLowShare) * sum_over_groups(l_run));
      f32x4 s0, s1;
      qk(tb, s0, s1);
      if (j + 1 < total) {
        cursor_next(sc, p, tpp);
        if (sc.b != cur.b) {
          load_q(sc.b);
          q_pending = true;
        }
      }
      s0 *= p.scale_log2;
      s1 *= p.scale_log2;
      const int nvalid = cur.Lr - cur.t * kTile;
      if (nvalid < kTile) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (4 * q4 + e >= nvalid) s0[e] = -INFINITY;
          if (16 + 4 * q4 + e >= nvalid) s1[e] = -INFINITY;
        }
      }
      causal_mask(p, cur, nvalid, head, q4, s0, s1, cfrom);
      // Online softmax over the tile's 32 scores of this lane's head (lazy rescale).  The
      // running maximum m_run (equal in the head's four lanes) moves only when a score
      // exceeds it by more than kRescaleSlack, which each lane can test on its own 8 scores:
      // the cross-lane maximum is taken only in a tile where some lane of the wave sees
      // such a score (the first of a piece, rarely later).  l_run is this lane's share of
      // the row sum; the four shares are added once, at the end of the piece.
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) { x[e] = s0[e]; x[e + 4] = s1[e]; }
      const float mloc = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                               fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      float alpha = 1.f;
      if (__any(mloc > m_run + kRescaleSlack)) {
        const float mh = max_over_groups(mloc);
        const float m_new = mh > m_run + kRescaleSlack ? mh : m_run;
        // no visible token yet (a causally masked row): nothing to weigh or rescale
        alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
        lo_thr += m_new == -INFINITY ? 0.f : m_run - m_new;  // log2(alpha)
        l_run *= alpha;
        m_run = m_new;
      }
      const bool none = m_run == -INFINITY;
      // (a row with no visible token has mloc - m_run = NaN: never flagged)
      const bool need_lo = cur.Lr <= kLowAllTokens || __any(mloc - m_run > lo_thr);
      if (q4 == 0) {
        s_alpha[par][l16][sb] = alpha;
        s_lo[par][l16][sb] = need_lo;
      }
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pr = none ? 0.f : fast_exp2(x[e] - m_run);
        l_run += pr;
        pb[e] = (__bf16)pr;
      }
      s_p[par][sb][lane] = pb;
      if (need_lo) {
        float lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[e] = (none ? 0.f : fast_exp2(x[e] - m_run)) - (float)pb[e];
        s_pl[par][sb][lane] = code_low_parts(lo);
      }
      if (cur.t == cur.ntile - 1 || j == total - 1) {
        bool whole;
        const int64_t row = piece_row(pc, cur, head_ok ? head : 0, whole);
        const float l_tot = sum_over_groups(l_run);
        if (q4 == 0) {
          // a row that saw no token of the piece: O = 0, LSE = -inf
          s_inv[par][l16][sb] = l_tot > 0.f ? 1.0f / l_tot : 0.f;
          if (head_ok)
            (whole ? p.out_lse : p.ws_lse)[row] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
        }
        pc.t0 = 0;
        pc.first = false;
        m_run = -INFINITY;
        l_run = 0.f;
      }
      // Every iteration ends at the barrier that starts the P.V waves' interval for
      // tile j (the P.V waves pass one barrier more: the one before this loop).
      if (q_pending) {
        wait_vmcnt_builtin<0>();
        q_pending = false;
      }
      wait_lgkm();
      wg_barrier();
    }
  } else {
    // ================================================================ P.V waves
    const int v = wave - kRoleWaves;    // dims kDims v .. kDims v + kDims - 1
    const bool copier = v < kCopyWaves;  // the first four P.V waves issue the tile copies

    // This lane's copies: LDS slot s = (k * 4 + v) * 64 + lane of a tile.
    uint32_t ld_off[kCopies];
#pragma unroll
    for (int k = 0; k < kCopies; ++k) {
      const int s = (k * kCopyWaves + v) * 64 + lane;
      const int row = s / kChunks;
      const int pos = s - row * kChunks;
      ld_off[k] = (uint32_t)(row * kRowBytes + (pos ^ row_swz(row)) * 16);
    }
    // V^T operand of dim block mm (dims kDims v + 16 mm ..): rows 4 q4 + l16 / 4 (+16),
    // chunk kDims v / 8 + 2 mm + (l16 % 4) / 2, byte half l16 % 2; the row swizzle
    // permutes chunks within aligned groups of 8.
    uint32_t vb[4];
    {
      const int r = 4 * q4 + (l16 >> 2);
      const int x = row_swz(r);
      const int h = (l16 & 3) >> 1;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        vb[m] = (uint32_t)(r * kRowBytes + 32 * (m ^ (x >> 1)) + 16 * (h ^ (x & 1)) + 8 * (l16 & 1) +
                           2 * PVC::kDims * v);
    }
    auto voff = [&](int mm) { return vb[mm & 3] + 128 * (mm >> 2); };

    Cursor lc = cur0;
    int lc_left = total;
    const uint8_t* src = nullptr;
    bool bad_page = false;
    auto next_src = [&]() {
      const int32_t page = checked_page(ld_const(lc.bt_row + lc.pk), p.num_cache_blocks, bad_page);
      src = p.k_cache + page * page_bytes + lc.sub * kTileBytes;
    };
    auto issue_tile = [&](int stage) {
      if (!copier) return;
#pragma unroll
      for (int k = 0; k < kCopies; ++k)
        copy16<kStream>(src, ld_off[k], lds_addr(lds + stage * kTileBytes + (k * kCopyWaves + v) * 1024));
      if (--lc_left > 0) {
        cursor_next(lc, p, tpp);
        next_src();
      }
    };
    // A copying wave's tile wait; a wave without copies has nothing in LDS to wait for.
    auto wait_tiles = [&]() {
      if (copier) wait_vmcnt_builtin<kCopies>();
    };

    f32x4 oacc[kDimBlocks][kHeadBlocks];
#pragma unroll
    for (int m = 0; m < kDimBlocks; ++m)
#pragma unroll
      for (int hb = 0; hb < kHeadBlocks; ++hb) oacc[m][hb] = f32x4{};

    Cursor pc_cur = cur0;
    Piece pc{pc_cur.t, true};

    // A finished piece is stored at the top of the next interval, before that
    // interval's copies: the tile wait at its end then covers the stores too, whatever
    // their number.
    bool pend = false;
    f32x4 pend_inv;
    float* pend_dst = nullptr;  // row of head hbase + l16; head block hb is 16 rows further
    auto flush_piece = [&]() {
      if (!pend) return;
#pragma unroll
      for (int hb = 0; hb < kHeadBlocks; ++hb) {
        if (hbase + 16 * hb + l16 < H) {
#pragma unroll
          for (int m = 0; m < kDimBlocks; ++m) {
            f32x4* dst = (f32x4*)(pend_dst + (int64_t)16 * hb * kDv + 16 * m);
            // With one head group the outputs and pieces also bypass the caches like the
            // page stream (B = 512 batch: ~4% faster calls); with several, the pieces of the
            // shared spans stay cached (non-temporal there was slower).
            if constexpr (kStream) __builtin_nontemporal_store(oacc[m][hb] * pend_inv[hb], dst);
            else *dst = oacc[m][hb] * pend_inv[hb];
          }
        }
#pragma unroll
        for (int m = 0; m < kDimBlocks; ++m) oacc[m][hb] = f32x4{};
      }
      pend = false;
    };

    // prologue: tiles 0 and 1 in flight; tile 0 landed before the first barrier
    if (copier) next_src();
    issue_tile(0);
    issue_tile(1);
    wait_tiles();
    wg_barrier();

    for (int i = -1; i < total; ++i) {
      flush_piece();
      issue_tile((i + 3) % kStages);  // past the span's end: the last tile again, unread
      if (i >= 0) {
        const Cursor cur = pc_cur;
        const int par = i & 1;
        const DCP_LDS uint8_t* tb = lds + (i % kStages) * kTileBytes;
        const int nvalid = cur.Lr - cur.t * kTile;
        if (nvalid < kTile) {
          // zero this wave's V dims of the rows past the request's end (its chunks form
          // whole swizzle groups, so no swizzle is needed)
          constexpr int kC = PVC::kChunksPerRow;
          const int n = (kTile - nvalid) * kC;
          for (int e = lane; e < n; e += 64)
            zero_lds16(lds_addr(tb + (nvalid + e / kC) * kRowBytes + (kC * v + e % kC) * 16));
        }
        const f32x4 alpha = *(const DCP_LDS f32x4*)&s_alpha[par][l16][0];
        // the head blocks whose tile takes the low parts of its weights (the same in every lane)
        const i32x4 lo_flags = *(const DCP_LDS i32x4*)&s_lo[par][l16][0];
        // (kept a vector value: a scalar copy would wait for this read before the pass below)
        const int lo_blocks = lo_flags[0] | lo_flags[1] << 1 | lo_flags[2] << 2 | lo_flags[3] << 3;
        bf16x8 pP[kHeadBlocks];
#pragma unroll
        for (int hb = 0; hb < kHeadBlocks; ++hb) pP[hb] = s_p[par][hb][lane];
        const bool moved = alpha[0] != 1.f || alpha[1] != 1.f || alpha[2] != 1.f || alpha[3] != 1.f;
        if (__any(moved)) {
#pragma unroll
          for (int m = 0; m < kDimBlocks; ++m)
#pragma unroll
            for (int hb = 0; hb < kHeadBlocks; ++hb) oacc[m][hb] *= alpha[hb];
        }
        // O^T += V^T P^T over the tile with the high parts of the weights
        u32x2 v1[kPfV], v2[kPfV];
#pragma unroll
        for (int m = 0; m < kPfV; ++m) {
          v1[m] = lds_read_tr16(tb + voff(m));
          v2[m] = lds_read_tr16(tb + voff(m) + 16 * kRowBytes);
        }
#pragma unroll
        for (int m = 0; m < kDimBlocks; ++m) {
          const bf16x8 a = join_tr16(v1[m % kPfV], v2[m % kPfV]);
          const int mn = m + kPfV;
          if (mn < kDimBlocks) {
            v1[m % kPfV] = lds_read_tr16(tb + voff(mn));
            v2[m % kPfV] = lds_read_tr16(tb + voff(mn) + 16 * kRowBytes);
          }
#pragma unroll
          for (int hb = 0; hb < kHeadBlocks; ++hb) oacc[m][hb] = mfma16x16x32(a, pP[hb], oacc[m][hb]);
        }
        // keep the V^T reads kPfV blocks ahead of the MFMAs (the scheduler would otherwise
        // sink them next to their use and expose the LDS latency block by block)
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPfV, 0);
#pragma unroll
        for (int m = 0; m < kDimBlocks - kPfV; ++m) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, kHeadBlocks, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kHeadBlocks * (kDimBlocks < kPfV ? kDimBlocks : kPfV), 0);
        if (lo_blocks) {
          // and with the low parts of the head blocks whose tile needs them: a second
          // pass over the V^T operands (kept apart so the common pass above keeps its
          // registers)
          u32x2 w1[kDimBlocks], w2[kDimBlocks];
#pragma unroll
          for (int m = 0; m < kDimBlocks; ++m) {
            w1[m] = lds_read_tr16(tb + voff(m));
            w2[m] = lds_read_tr16(tb + voff(m) + 16 * kRowBytes);
          }
#pragma unroll
          for (int hb = 0; hb < kHeadBlocks; ++hb) {
            if (lo_blocks >> hb & 1) {
              const bf16x8 pL = decode_low_parts(s_pl[par][hb][lane]);
#pragma unroll
              for (int m = 0; m < kDimBlocks; ++m) oacc[m][hb] = mfma16x16x32(join_tr16(w1[m], w2[m]), pL, oacc[m][hb]);
            }
          }
        }
        if (cur.t == cur.ntile - 1 || i == total - 1) {
          // 1/l of every head leaves LDS now: the next tile of this parity overwrites it
          pend_inv = *(const DCP_LDS f32x4*)&s_inv[par][l16][0];
          bool whole;
          const int64_t row = piece_row(pc, cur, hbase + l16, whole);
          pend_dst = (whole ? p.out_o : p.ws_o) + row * kDv + PVC::kDims * v + 4 * q4;
          pend = true;
          pc.t0 = 0;
          pc.first = false;
        }
        if (i + 1 < total) cursor_next(pc_cur, p, tpp);
      }
      if (i + 1 < total) {
        // tile i+2 has landed once only the copies of tile i+3 are outstanding
        wait_tiles();
        wg_barrier();
      }
    }
    flush_piece();
    if (bad_page && lane == 0) report_error(p.ws_err, kErrPageId);
    // No copy may still be landing in this work-group's LDS when it exits.
    wait_vmcnt_builtin<0>();
  }
}

}  // namespace mla

hipError_t launch_mla_partial(const PartialParams& p, hipStream_t stream) {
  constexpr int kWidePV = mla::wide::kPVWaves;
  const int grid = p.part.num_parts * p.num_head_groups;
  if (mla_heads_per_group(p.num_q_heads) == 32)
    hipLaunchKernelGGL(mla::mla_partial_kernel<1>, dim3(grid), dim3(128), 0, stream, p);
  else if (p.num_head_groups == 1)
    hipLaunchKernelGGL((mla::mla_partial_wide_kernel<true, kWidePV>), dim3(grid),
                       dim3(mla::wide::PV<kWidePV>::kThreads), 0, stream, p);
  else  // the head groups of a span share its pages through L2
    hipLaunchKernelGGL((mla::mla_partial_wide_kernel<false, kWidePV>), dim3(grid),
                       dim3(mla::wide::PV<kWidePV>::kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dcp
