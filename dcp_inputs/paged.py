"""Device-resident paged KV caches for a synthetic workload (GPU harness).

Builds, for one rank, the rank-local page pool, its block table and the query,
filled on the device by the seeded generator.  Which tokens a rank holds and in
which local order is taken from the library's own host shard map
(``dcp_shard_map`` / ``dcp_shard_global``); this module adds no arithmetic of
its own beyond page bookkeeping.  The float64 oracle never imports it: it
regenerates its inputs from (seed, logical row) and enumerates shard ownership
itself.

Layout:
* every pool page not holding a valid token row is filled with bf16 NaN (the tail
  slots of each request's last page and a dedicated poison page);
* block-table entries past a request's last local page point at the poison page;
* physical page ids are a seeded permutation, so a request's pages are scattered.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

import dcp_inputs as di
import decode_attention_sequence_paged_amd as dcp


@dataclass
class RankCache:
    rank: int
    local_lens: np.ndarray          # int64 [B]
    block_table: torch.Tensor       # int32 [B, max_blocks] (device)
    k_cache: torch.Tensor           # bf16 pool (device)
    v_cache: Optional[torch.Tensor]  # GQA only
    poison_page: int

    @property
    def total_local(self) -> int:
        return int(self.local_lens.sum())

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


def device_query(wl, seed: Optional[int] = None, census: bool = False) -> torch.Tensor:
    seed = wl.seed if seed is None else seed
    q = torch.empty((wl.batch, wl.num_q_heads, wl.qk_dim), dtype=torch.bfloat16, device="cuda")
    if census:
        q.zero_()
        return q
    n = wl.batch * wl.num_q_heads
    idx = torch.arange(n, dtype=torch.int64, device="cuda")
    di.device_fill_rows(q.view(torch.int16), idx, idx, wl.qk_dim, seed, di.STREAM_Q,
                        hip_stream=torch.cuda.current_stream().cuda_stream)
    return q


def build_rank_cache(wl, rank: int, seed: Optional[int] = None, census: bool = False,
                     lengths: Optional[np.ndarray] = None, extra_blocks: int = 0) -> RankCache:
    """Rank ``rank``'s page pool for workload ``wl`` (N = wl.dcp_size, I = wl.interleave).

    census=True writes, instead of seeded normals, the census rows: element d of the
    row of global token t is bit d of t (d < 24) -- see dcp_inputs.census_rows_numpy.
    """
    seed = wl.seed if seed is None else seed
    seq_lens = np.asarray(wl.lengths if lengths is None else lengths, dtype=np.int64)
    N, I, bs = wl.dcp_size, wl.interleave, wl.block_size
    local, _, _ = dcp.dcp_shard_map(seq_lens.astype(np.int32), N, I, rank)
    local = local.astype(np.int64)
    pages = (local + bs - 1) // bs
    total_pages = int(pages.sum()) + 1
    perm = di.page_permutation(total_pages, seed, salt=rank)
    poison = int(perm[-1])
    max_blocks = max(1, int(pages.max()) if pages.size else 1) + extra_blocks
    bt = np.full((seq_lens.size, max_blocks), poison, dtype=np.int32)
    off = 0
    for b in range(seq_lens.size):
        bt[b, :pages[b]] = perm[off:off + pages[b]]
        off += int(pages[b])

    # every valid local token: (destination row in the pool, logical row id / census id)
    dst_rows, row_ids = [], []
    for b in range(seq_lens.size):
        if local[b] == 0:
            continue
        j = np.arange(local[b], dtype=np.int64)
        t = dcp.dcp_shard_global(j, N, I, rank)
        dst_rows.append(bt[b, j // bs].astype(np.int64) * bs + j % bs)
        row_ids.append(t if census else (np.int64(b) << di.ROW_T_BITS) + t)
    dst = torch.from_numpy(np.concatenate(dst_rows) if dst_rows else np.zeros(0, np.int64)).cuda()
    ids = torch.from_numpy(np.concatenate(row_ids) if row_ids else np.zeros(0, np.int64)).cuda()
    stream = torch.cuda.current_stream().cuda_stream
    mode = 1 if census else 0

    if wl.kind == "mla":
        pool = torch.empty((total_pages, bs, wl.qk_dim), dtype=torch.bfloat16, device="cuda")
        di.device_fill_value(pool.view(torch.int16), di.BF16_NAN_BITS, hip_stream=stream)
        di.device_fill_rows(pool.view(torch.int16), dst, ids, wl.qk_dim, seed, di.STREAM_K,
                            mode=mode, hip_stream=stream)
        vpool = None
    else:
        H = wl.num_kv_heads
        pool = torch.empty((total_pages, bs, H, wl.qk_dim), dtype=torch.bfloat16, device="cuda")
        vpool = torch.empty((total_pages, bs, H, wl.v_dim), dtype=torch.bfloat16, device="cuda")
        di.device_fill_value(pool.view(torch.int16), di.BF16_NAN_BITS, hip_stream=stream)
        di.device_fill_value(vpool.view(torch.int16), di.BF16_NAN_BITS, hip_stream=stream)
        g = torch.arange(H, dtype=torch.int64, device="cuda")
        dst_g = (dst[:, None] * H + g[None, :]).reshape(-1)
        if census:
            ids_g = ids[:, None].expand(-1, H).reshape(-1).contiguous()
        else:
            ids_g = (ids[:, None] * H + g[None, :]).reshape(-1)
        di.device_fill_rows(pool.view(torch.int16), dst_g, ids_g, wl.qk_dim, seed, di.STREAM_K,
                            mode=mode, hip_stream=stream)
        di.device_fill_rows(vpool.view(torch.int16), dst_g, ids_g, wl.v_dim, seed, di.STREAM_V,
                            mode=mode, hip_stream=stream)
    return RankCache(rank, local, torch.from_numpy(bt).cuda(), pool, vpool, poison)


def desc_for(wl) -> "dcp.AttnDesc":
    kind = dcp.DCP_KV_MLA_LATENT if wl.kind == "mla" else dcp.DCP_KV_GQA
    return dcp.attn_desc(kind, wl.num_q_heads, wl.num_kv_heads, wl.qk_dim, wl.v_dim, wl.block_size,
                         wl.softmax_scale)


def workspace_for(wl, num_partitions: int = 0, q_len: int = 1) -> torch.Tensor:
    """A zero-initialised workspace for the workload's partial calls."""
    nbytes = dcp.dcp_decode_workspace_size_mtp(desc_for(wl), q_len, wl.batch, num_partitions)
    if nbytes == 0:
        raise ValueError("unsupported workload shape for %s" % wl.name)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dcp.dcp_workspace_init(ws)
    return ws


def run_partial(wl, rc: RankCache, q: torch.Tensor, seq_lens_dev: torch.Tensor, out_o, out_lse,
                workspace, num_partitions: int = 0, stream=None) -> None:
    dcp.dcp_decode_partial(desc_for(wl), q, rc.k_cache, rc.v_cache, rc.block_table, seq_lens_dev,
                           rc.rank, wl.dcp_size, wl.interleave, workspace, out_o, out_lse,
                           num_partitions=num_partitions, stream=stream)
