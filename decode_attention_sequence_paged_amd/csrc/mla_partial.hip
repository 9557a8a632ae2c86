// MLA partial decode attention over one rank's shard of a paged latent KV cache.
//
// What it computes (vLLM blog "Efficient Decode Context Parallelism with vLLM for
// Long Context Workloads", Sec. 4.1 "Compute" and Sec. 5.3 "MLA Backend"): every
// query head attends the rank's local latent rows; K is the whole 576-dim row and
// V its first 512 entries (the weight-absorbed form, where the query is already in
// the latent space).  Output: normalised partial O [B,H,512] and LSE [B,H].
//
// Design for gfx950:
//  * A work-group owns 64 query heads (NPAIR = 2) or 32 (NPAIR = 1) and a
//    token-balanced span of the rank's tiles (32 tokens each).  Every latent row is
//    read from HBM once per head group and used as both K and V.
//  * Tiles stream HBM -> LDS with 16-byte direct-to-LDS loads through an NSTAGE ring;
//    no VGPRs are spent on staging, so the loads of the next stages stay in flight
//    while the current tile is computed.  Row chunks are rotated by the row index in
//    LDS so the MFMA operand reads of 32 rows hit distinct banks.
//  * Waves come in pairs that share 32 heads.  QK^T (contraction 576) is split by
//    dimension halves across the pair (each wave keeps its 32 x 288 slice of q in
//    VGPRs); the two 32x32 fp32 score halves are summed through LDS.  PV is split by
//    output halves (each wave accumulates O^T for 256 of the 512 dims).
//  * Both contractions use v_mfma_f32_32x32x16_bf16.  S^T = K Q^T puts tokens on the
//    MFMA rows and heads on the columns, so each lane's softmax statistics belong to
//    one head; the S^T accumulator, converted to bf16, is directly the B operand of
//    O^T += V^T P^T.  V^T comes from LDS through the transposing ds_read_b64_tr_b16.
//  * Online softmax in base 2 with fp32 statistics; the O accumulator is rescaled
//    only when some head's running maximum moved.
#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {
namespace mla {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;        // 1152
constexpr int kChunks = kRowBytes / 16;    // 72 16-byte chunks per row
constexpr int kTile = 32;                  // tokens per tile
constexpr int kTileBytes = kTile * kRowBytes;  // 36864
constexpr int kStages = 3;
constexpr int kXchgBytes = 64 * 16 * 4;    // one wave's 32x32 fp32 score half
constexpr int kQSteps = kDqk / 2 / 16;     // 18 k-steps of 16 dims per half

// LDS byte offset of 16-byte chunk c of tile row `row` (rotated placement).
__device__ __forceinline__ int chunk_off(int row, int c) {
  int pc = c + row;
  pc = pc >= kChunks ? pc - kChunks : pc;
  return row * kRowBytes + pc * 16;
}

template <int NPAIR>
struct Cfg {
  static constexpr int kWaves = 2 * NPAIR;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kHeads = 32 * NPAIR;
  static constexpr int kLoads = kTile * kChunks / kThreads;  // DMA loads per thread per tile
  static_assert(kTile * kChunks % kThreads == 0, "tile must split evenly");
  static constexpr int kLdsBytes = kStages * kTileBytes + kWaves * kXchgBytes;
};

template <int NPAIR>
__global__ __launch_bounds__(128 * NPAIR, 1) void mla_partial_kernel(PartialParams p) {
  using C = Cfg<NPAIR>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLdsBytes];
  __shared__ int64_t s_scan[C::kThreads];
  __shared__ int64_t s_loc[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int pair = wave >> 1;
  const int half = wave & 1;     // QK dims [288*half, +288); O dims [256*half, +256)
  const int l32 = lane & 31;
  const int hi = lane >> 5;      // 0/1: which half of the wave

  int64_t w;
  int hg;
  block_to_span(p.part.num_parts, p.num_head_groups, &w, &hg);
  const bool write_prefix = (w == 0 && hg == 0);
  SpanLoc loc = locate_span<C::kThreads>(p.part, w, write_prefix ? p.ws_prefix : nullptr, s_scan,
                                         s_loc);
  if (loc.start >= loc.end) return;

  const int H = p.num_q_heads;
  const int head = hg * C::kHeads + pair * 32 + l32;   // this lane's head (S^T column)
  const bool head_ok = head < H;

  DCP_LDS uint8_t* lds = (DCP_LDS uint8_t*)smem;
  DCP_LDS uint8_t* xbuf = lds + kStages * kTileBytes;

  // Per-lane source offsets of the DMA loads inside a tile (row-major 1152-byte rows).
  int ld_row[C::kLoads];
  int ld_off[C::kLoads];
#pragma unroll
  for (int k = 0; k < C::kLoads; ++k) {
    const int s = (k * C::kWaves + wave) * 64 + lane;   // LDS slot of this lane's chunk
    const int row = s / kChunks;
    const int pc = s - row * kChunks;
    int c = pc - row;
    c = c < 0 ? c + kChunks : c;
    ld_row[k] = row;
    ld_off[k] = row * kRowBytes + c * 16;
  }

  int64_t remaining = loc.end - loc.start;
  int b = loc.b0;
  int64_t toff = loc.off0;
  bool first_piece = true;

  while (remaining > 0) {
    const int64_t Lr = part_local_len(p.part, b);
    const int64_t ntile = (Lr + kTile - 1) / kTile;
    if (ntile == 0) { ++b; continue; }
    const int64_t n = (ntile - toff) < remaining ? (ntile - toff) : remaining;
    const bool whole = (toff == 0 && n == ntile);
    const int32_t* bt_row = p.block_table + (int64_t)b * p.max_blocks_per_seq;

    // ---- query slice of this wave: q[b, head, 288*half + 16*s + 8*hi .. +7]
    bf16x8 qreg[kQSteps];
    {
      const uint16_t* qp = p.q + ((int64_t)b * H + (head_ok ? head : 0)) * kDqk + 288 * half + 8 * hi;
#pragma unroll
      for (int s = 0; s < kQSteps; ++s) {
        bf16x8 v = *(const bf16x8*)(qp + 16 * s);
        if (!head_ok) v = bf16x8{};
        qreg[s] = v;
      }
    }

    auto issue_tile = [&](int64_t t_local, int stage) {
      const int64_t tok0 = t_local * kTile;
      const int32_t page = clamp_page(ld_const(bt_row + tok0 / p.block_size), p.num_cache_blocks);
      const int64_t slot0 = tok0 % p.block_size;
      const int nvalid = (int)((Lr - tok0) < kTile ? (Lr - tok0) : kTile);
      const uint8_t* base = p.k_cache + ((int64_t)page * p.block_size + slot0) * kRowBytes;
      DCP_LDS uint8_t* dst = lds + stage * kTileBytes;
#pragma unroll
      for (int k = 0; k < C::kLoads; ++k) {
        int off = ld_off[k];
        if (ld_row[k] >= nvalid) off -= (ld_row[k] - (nvalid - 1)) * kRowBytes;  // replicate last row
        dma16(base + off, dst + (k * C::kWaves + wave) * 1024);
      }
    };

    f32x16 oacc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) oacc[m] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    // prologue
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
      if (s < n) issue_tile(toff + s, s);

    for (int64_t i = 0; i < n; ++i) {
      if (i + kStages - 2 < n) wait_vmcnt<C::kLoads * (kStages - 2)>();
      else wait_vmcnt<0>();
      wg_barrier();
      if (i + kStages - 1 < n) issue_tile(toff + i + kStages - 1, (int)((i + kStages - 1) % kStages));

      const DCP_LDS uint8_t* tb = lds + (int)(i % kStages) * kTileBytes;
      const int64_t tok0 = (toff + i) * kTile;
      const int nvalid = (int)((Lr - tok0) < kTile ? (Lr - tok0) : kTile);

      // ---- S^T half = K[:, half dims] . Q^T   (rows = tokens, cols = heads)
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int s = 0; s < kQSteps; ++s) {
        const int c = 36 * half + 2 * s + hi;
        const bf16x8 a = *(const DCP_LDS bf16x8*)(tb + chunk_off(l32, c));
        sacc = mfma32x32x16(a, qreg[s], sacc);
      }

      // ---- sum the two dimension halves of the pair through LDS
      DCP_LDS f32x4* xw = (DCP_LDS f32x4*)(xbuf + wave * kXchgBytes);
      DCP_LDS f32x4* xp = (DCP_LDS f32x4*)(xbuf + (wave ^ 1) * kXchgBytes);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xw[j * 64 + lane] = f32x4{sacc[4 * j], sacc[4 * j + 1], sacc[4 * j + 2], sacc[4 * j + 3]};
      wg_barrier();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 o = xp[j * 64 + lane];
        sacc[4 * j] += o[0];
        sacc[4 * j + 1] += o[1];
        sacc[4 * j + 2] += o[2];
        sacc[4 * j + 3] += o[3];
      }

      // ---- online softmax (base 2).  Lane holds head `head`, tokens 8(r/4)+4*hi+(r%4).
      float x[16];
      float mloc = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = 8 * (r >> 2) + 4 * hi + (r & 3);
        x[r] = tok < nvalid ? sacc[r] * p.scale_log2 : -INFINITY;
        mloc = fmaxf(mloc, x[r]);
      }
      mloc = fmaxf(mloc, shfl_xor_f(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = fast_exp2(m_run - m_new);
      float lsum = 0.f;
      bf16x8 pb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = fast_exp2(x[r] - m_new);
        lsum += pr;
        pb[r >> 3][r & 7] = (__bf16)pr;
      }
      lsum += shfl_xor_f(lsum, 32);
      l_run = l_run * alpha + lsum;
      m_run = m_new;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int m = 0; m < 8; ++m) oacc[m] *= alpha;
      }

      // ---- O^T[256*half .. +256, heads] += V^T P^T over the 32 tokens
      const int grp = (lane >> 4) & 1;
      const int sl = lane & 15;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int d0 = 256 * half + 32 * m + 16 * grp + 4 * (sl & 3);   // source lane's 4 dims
          const int c = d0 >> 3;
          const int hb = (d0 & 4) * 2;                                    // byte offset in chunk
          const int r1 = 16 * ks + 4 * hi + (sl >> 2);
          const int r2 = r1 + 8;
          const u32x2 v1 = lds_read_tr16(tb + chunk_off(r1, c) + hb);
          const u32x2 v2 = lds_read_tr16(tb + chunk_off(r2, c) + hb);
          const bf16x8 a = join_tr16(v1, v2);
          oacc[m] = mfma32x32x16(a, pb[ks], oacc[m]);
        }
      }
    }
    wg_barrier();  // every wave is done with the ring and the exchange buffers

    // ---- epilogue: normalise and store.  oacc[m] lane reg r -> dim 256*half + 32m + 8(r/4) + 4*hi + r%4
    if (head_ok) {
      const float inv = 1.0f / l_run;
      const float lse = (m_run + fast_log2(l_run)) * kLn2;
      const int64_t slot = 2 * w + (first_piece ? 0 : 1);
      float* orow = whole ? p.out_o + ((int64_t)b * H + head) * kDv
                          : p.ws_o + (slot * H + head) * kDv;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 256 * half + 32 * m + 8 * j + 4 * hi;
          *(f32x4*)(orow + d) = f32x4{oacc[m][4 * j] * inv, oacc[m][4 * j + 1] * inv,
                                      oacc[m][4 * j + 2] * inv, oacc[m][4 * j + 3] * inv};
        }
      }
      if (half == 0 && hi == 0) {
        if (whole) p.out_lse[(int64_t)b * H + head] = lse;
        else p.ws_lse[slot * H + head] = lse;
      }
    }

    remaining -= n;
    first_piece = false;
    ++b;
    toff = 0;
  }
}

}  // namespace mla

int mla_heads_per_group(int num_q_heads) { return num_q_heads <= 32 ? 32 : 64; }

hipError_t launch_mla_partial(const PartialParams& p, hipStream_t stream) {
  const int grid = p.part.num_parts * p.num_head_groups;
  if (mla_heads_per_group(p.num_q_heads) == 32)
    hipLaunchKernelGGL(mla::mla_partial_kernel<1>, dim3(grid), dim3(128), 0, stream, p);
  else
    hipLaunchKernelGGL(mla::mla_partial_kernel<2>, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dcp
