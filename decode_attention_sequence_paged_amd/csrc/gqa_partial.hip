// GQA partial decode attention over one rank's shard of a paged K/V cache.
//
// What it computes (vLLM blog "Efficient Decode Context Parallelism with vLLM for
// Long Context Workloads", Sec. 4.1 "Compute" and Sec. 5.4 "GQA Backend"): each KV
// head is shared by its group of G = H / Hkv query heads (query head h reads KV
// head h / G).  Output: normalised partial O [B,H,128] and LSE [B,H] over the
// rank's tokens.
//
// Design for gfx950: one wave per KV head (up to 4 KV heads per work-group, so a
// token's K row slice and V row slice of the group are contiguous 256*W bytes),
// tiles of 32 tokens streamed HBM -> LDS by direct 16-byte loads into a two-stage
// ring, v_mfma_f32_16x16x32_bf16 for S^T = K Q^T (16 heads on the columns) and for
// O^T += V^T P^T (V^T through the transposing LDS read), online softmax in base 2.
#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {
namespace gqa {

constexpr int kD = 128;
constexpr int kHeadBytes = kD * 2;  // 256
constexpr int kTile = 32;
constexpr int kStages = 2;

template <int KVW>
struct Cfg {
  static constexpr int kThreads = 64 * KVW;
  static constexpr int kRowBytes = KVW * kHeadBytes;       // one token's slice of the group
  static constexpr int kChunks = kRowBytes / 16;           // 16 * KVW
  static constexpr int kHalfBytes = kTile * kRowBytes;     // K (or V) part of a stage
  static constexpr int kStageBytes = 2 * kHalfBytes;
  static constexpr int kLoads = kTile * kChunks / kThreads;  // 8 per thread for K, 8 for V
  static constexpr int kLdsBytes = kStages * kStageBytes;
};

// LDS byte offset of 16-byte chunk c of tile row `row`: chunks are rotated by the
// row index (modulo the power-of-two chunk count) so that 16 rows read at the same
// logical chunk hit different banks.
template <int KVW>
__device__ __forceinline__ int chunk_off(int row, int c) {
  constexpr int CH = Cfg<KVW>::kChunks;
  static_assert((CH & (CH - 1)) == 0, "chunk count must be a power of two");
  return row * Cfg<KVW>::kRowBytes + ((c + row) & (CH - 1)) * 16;
}

template <int KVW>
__global__ __launch_bounds__(64 * KVW, 1) void gqa_partial_kernel(PartialParams p) {
  using C = Cfg<KVW>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLdsBytes];
  __shared__ int64_t s_scan[C::kThreads];
  __shared__ int64_t s_loc[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int l16 = lane & 15;
  const int q4 = lane >> 4;  // 0..3

  int64_t w;
  int hg;
  block_to_span(p.part.num_parts, p.num_head_groups, &w, &hg);
  const bool write_prefix = (w == 0 && hg == 0);
  SpanLoc loc = locate_span<C::kThreads>(p.part, w, write_prefix ? p.ws_prefix : nullptr, s_scan,
                                         s_loc);
  if (loc.start >= loc.end) return;

  const int H = p.num_q_heads;
  const int Hkv = p.num_kv_heads;
  const int G = H / Hkv;
  const int g0 = hg * KVW;             // first KV head of the work-group
  const int g = g0 + wave;             // this wave's KV head
  const int head = g * G + l16;        // this lane's query head (S^T column)
  const bool head_ok = l16 < G;

  DCP_LDS uint8_t* lds = (DCP_LDS uint8_t*)smem;

  int ld_row[C::kLoads];
  int ld_off[C::kLoads];
#pragma unroll
  for (int k = 0; k < C::kLoads; ++k) {
    const int s = (k * KVW + wave) * 64 + lane;
    const int row = s / C::kChunks;
    const int pc = s - row * C::kChunks;
    ld_row[k] = row;
    ld_off[k] = ((pc - row) & (C::kChunks - 1)) * 16;   // inverse of chunk_off's rotation
  }
  const int64_t row_stride = (int64_t)Hkv * kHeadBytes;  // bytes between token rows in the pool

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

    // q[b, head, 32*s + 8*q4 .. +7]
    bf16x8 qreg[4];
    {
      const uint16_t* qp = p.q + ((int64_t)b * H + (head_ok ? head : g * G)) * kD + 8 * q4;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 v = *(const bf16x8*)(qp + 32 * s);
        if (!head_ok) v = bf16x8{};
        qreg[s] = v;
      }
    }

    auto issue_tile = [&](int64_t t_local, int stage) {
      const int64_t tok0 = t_local * kTile;
      const int nvalid = (int)((Lr - tok0) < kTile ? (Lr - tok0) : kTile);
      const int32_t page_lo = clamp_page(ld_const(bt_row + tok0 / p.block_size), p.num_cache_blocks);
      int32_t page_hi = page_lo;
      if (nvalid > 16)
        page_hi = clamp_page(ld_const(bt_row + (tok0 + 16) / p.block_size), p.num_cache_blocks);
      DCP_LDS uint8_t* kdst = lds + stage * C::kStageBytes;
      DCP_LDS uint8_t* vdst = kdst + C::kHalfBytes;
#pragma unroll
      for (int k = 0; k < C::kLoads; ++k) {
        const int row = ld_row[k] < nvalid ? ld_row[k] : nvalid - 1;
        const int64_t tok = tok0 + row;
        const int32_t page = row < 16 ? page_lo : page_hi;
        const int64_t off = ((int64_t)page * p.block_size + tok % p.block_size) * row_stride +
                            (int64_t)g0 * kHeadBytes + ld_off[k];
        dma16(p.k_cache + off, kdst + (k * KVW + wave) * 1024);
        dma16(p.v_cache + off, vdst + (k * KVW + wave) * 1024);
      }
    };

    f32x4 oacc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) oacc[m] = f32x4{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    issue_tile(toff, 0);
    for (int64_t i = 0; i < n; ++i) {
      wait_vmcnt<0>();
      wg_barrier();
      if (i + 1 < n) issue_tile(toff + i + 1, (int)((i + 1) & 1));

      const DCP_LDS uint8_t* kb = lds + (int)(i & 1) * C::kStageBytes;
      const DCP_LDS uint8_t* vb = kb + C::kHalfBytes;
      const int64_t tok0 = (toff + i) * kTile;
      const int nvalid = (int)((Lr - tok0) < kTile ? (Lr - tok0) : kTile);

      // S^T [32 tokens x 16 heads] as two 16x16 tiles
      f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int c = wave * 16 + 4 * s + q4;
          const bf16x8 a = *(const DCP_LDS bf16x8*)(kb + chunk_off<KVW>(16 * mt + l16, c));
          sacc[mt] = mfma16x16x32(a, qreg[s], sacc[mt]);
        }
      }

      // online softmax; lane holds head l16, tokens 16*mt + 4*q4 + r
      float x[8];
      float mloc = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tok = 16 * (j >> 2) + 4 * q4 + (j & 3);
        x[j] = tok < nvalid ? sacc[j >> 2][j & 3] * p.scale_log2 : -INFINITY;
        mloc = fmaxf(mloc, x[j]);
      }
      mloc = fmaxf(mloc, shfl_xor_f(mloc, 16));
      mloc = fmaxf(mloc, shfl_xor_f(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = fast_exp2(m_run - m_new);
      float lsum = 0.f;
      bf16x8 pb;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pr = fast_exp2(x[j] - m_new);
        lsum += pr;
        pb[j] = (__bf16)pr;
      }
      lsum += shfl_xor_f(lsum, 16);
      lsum += shfl_xor_f(lsum, 32);
      l_run = l_run * alpha + lsum;
      m_run = m_new;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int m = 0; m < 8; ++m) oacc[m] *= alpha;
      }

      // O^T [128 dims x 16 heads] += V^T [128 x 32 tokens] P^T [32 x 16]
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int d0 = 16 * m + 4 * (l16 & 3);      // source lane's 4 dims
        const int c = wave * 16 + (d0 >> 3);
        const int hb = (d0 & 4) * 2;
        const int r1 = 4 * q4 + (l16 >> 2);
        const u32x2 v1 = lds_read_tr16(vb + chunk_off<KVW>(r1, c) + hb);
        const u32x2 v2 = lds_read_tr16(vb + chunk_off<KVW>(r1 + 16, c) + hb);
        const bf16x8 a = join_tr16(v1, v2);
        oacc[m] = mfma16x16x32(a, pb, oacc[m]);
      }
    }
    wg_barrier();

    // epilogue: oacc[m] lane reg r -> dim 16m + 4*q4 + r, head l16
    if (head_ok) {
      const float inv = 1.0f / l_run;
      const float lse = (m_run + fast_log2(l_run)) * kLn2;
      const int64_t slot = 2 * w + (first_piece ? 0 : 1);
      float* orow = whole ? p.out_o + ((int64_t)b * H + head) * kD : p.ws_o + (slot * H + head) * kD;
#pragma unroll
      for (int m = 0; m < 8; ++m)
        *(f32x4*)(orow + 16 * m + 4 * q4) = oacc[m] * inv;
      if (q4 == 0) {
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

}  // namespace gqa

int gqa_kv_heads_per_group(int num_kv_heads) {
  return num_kv_heads % 4 == 0 ? 4 : (num_kv_heads % 2 == 0 ? 2 : 1);
}

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
