"""Benchmark of one decode-attention layer under Decode Context Parallelism on one GPU.

A step is the whole hot path for one decode batch: the partial attention of every
rank of the DCP group (ranks 0..N-1 run one after another on this GPU, each over
its own sequence shard of the paged KV cache) followed by the N-way LSE merge.
Inputs (query, every rank's page pool and block table) are resident in HBM
before timing starts.

Printed as one JSON line:
  value            KV bytes of all ranks / step time (GB/s): whole-job throughput
  ms_per_step      wall time of one step (K steps bracketed by synchronize)
  rank0_kv_gbps    local-shard KV GB/s of rank 0's partial call (HIP events, median)
  roofline         the partial-attention call against the 8 TB/s HBM peak
  cpu_baseline     the float64 oracle on the host cores, per-rank partials of the batch
  hbm_read_probe   attainable HBM read bandwidth of plain streaming loads on this device

With --bands it instead prints one JSON line with rank 0's partial-call bandwidth for
each request-length band of the pages' comparison by sequence length (<32k, 32-64k,
64-128k, 128-200k, >=200k tokens): the long-context MLA shape with requests drawn from
the synthetic mix restricted to the band, as many as give rank 0 about 1.25M tokens.

With --next it instead prints one JSON line timing the steps next to the hot path on the
long-context MLA batch: the partial calls of ranks 0..3 for 1, 2 and 4 query tokens per
request (multi-token decode queries, causal by global position; also on the GQA batch,
all four ranks), the append of every request's newest latent row into its owner rank's
page (all N ranks' calls), and the merge as per-rank steps (global LSE from the gathered
LSEs, local rescale with fp32 or bf16 transport, one rank's head slice of the sum) beside
the fused N-way merge.  Call times there are medians over the calls, events around every
call, no synchronisation between the calls.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "local-shard decode-attn KV GB/s & % of HBM peak; decode steps/s per batch"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "partial_traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None,
                    help="workload name (default: mla_c512; with --next: mla_long_b128)")
    ap.add_argument("--partitions", type=int, default=0, help="work partitions per head group (0 = default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the other workloads' figures (per_config)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of host work (oracle math + input regeneration) for the CPU baseline")
    ap.add_argument("--bands", action="store_true",
                    help="rank-0 partial bandwidth per request-length band instead of the step")
    ap.add_argument("--next", action="store_true",
                    help="time the steps next to the hot path (multi-token queries, KV append, "
                         "per-rank merge steps) instead of the step")
    ap.add_argument("--copy-probe-bytes", type=int, default=0,
                    help="before timing, run one plain device-to-device copy of this many bytes "
                         "(a reference for scaling the HBM byte counters of a profiler run)")
    return ap.parse_args()


def single_kernel_call(wl) -> bool:
    """Whether a partial call of this workload is one kernel launch (requests split between
    work partitions merged inside the kernel) or two (a split-K reduce kernel follows)."""
    return False


def describe(wl) -> str:
    if wl.kind == "mla":
        kv = "576-dim latent KV (V = first 512)"
    else:
        kv = "%d KV heads of %d+%d dims" % (wl.num_kv_heads, wl.qk_dim, wl.v_dim)
    return ("%s: %s decode, B=%d, %d query heads, %s, pages of %d tokens, N=%d ranks, "
            "interleave I=%d, lengths median %d max %d; all N ranks' partials + N-way merge per step"
            % (wl.name, wl.kind.upper(), wl.batch, wl.num_q_heads, kv, wl.block_size, wl.dcp_size,
               wl.interleave, int(np.median(wl.lengths)), int(max(wl.lengths))))


KERNEL_SOURCES = ("mla_partial.hip", "gqa_partial.hip", "reduce.hip", "dcp_device.h", "dcp_params.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_sequence_paged_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per dcp_decode_partial call from the committed rocprofv3 counter runs,
    if they were taken on this workload and on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    w = t.get("workloads", {}).get(workload)
    return None if w is None else w.get("hbm_bytes_per_launch")


def cpu_baseline(wl, budget_s: float):
    """Time the float64 oracle on the host: per-rank partial attention of the workload's
    requests, rank 0's requests in batch order, then rank 1's, ..., until about
    ``budget_s`` seconds of host work (attention math plus input regeneration) are spent.
    Only the attention math is timed for the rate."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    tokens = 0
    t_math = t_gen = 0.0
    done = []  # (rank, requests)
    for r in range(wl.dcp_size):
        n_req = 0
        for b in range(wl.batch):
            toks = oracle.rank_tokens(int(wl.lengths[b]), wl.dcp_size, wl.interleave, r)
            t0 = time.perf_counter()
            q, K, V = oracle.request_inputs(wl, b, toks)
            t1 = time.perf_counter()
            oracle.attention(q, K, V, wl.softmax_scale)
            t2 = time.perf_counter()
            t_gen += t1 - t0
            t_math += t2 - t1
            tokens += toks.size
            n_req += 1
            del q, K, V
            if t_math + t_gen >= budget_s:
                break
        done.append((r, n_req))
        if t_math + t_gen >= budget_s:
            break
    kv_bytes = tokens * (wl.qk_dim * 2 if wl.kind == "mla" else wl.num_kv_heads * (wl.qk_dim + wl.v_dim) * 2)
    sample = "; ".join("rank %d: requests 0..%d of %d" % (r, n - 1, wl.batch) for r, n in done)
    return {
        "value": round(kv_bytes / t_math / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": "per-rank partial attention (float64 numpy, %d BLAS threads) of %s (%d local tokens); "
                  "%.3g s of attention math timed, input regeneration (%.3g s) excluded; rate in "
                  "bf16-KV bytes per second" % (threads, sample, tokens, t_math, t_gen),
        "tokens_per_s": round(tokens / t_math, 1),
    }


def run_bands(args):
    """Rank 0's dcp_decode_partial call per length band (HIP events around each call)."""
    import torch
    import dcp_inputs as di
    import decode_attention_sequence_paged_amd as dcp
    from dcp_inputs import paged

    dcp.lib()
    torch.cuda.set_device(0)
    rows = []
    for lo, hi in di.LENGTH_BANDS:
        wl = di.band_workload(lo, hi)
        q = paged.device_query(wl)
        sl = torch.tensor(np.asarray(wl.lengths, dtype=np.int32), device="cuda")
        rc = paged.build_rank_cache(wl, 0)
        ws = paged.workspace_for(wl)
        o = torch.empty((wl.batch, wl.num_q_heads, wl.v_dim), device="cuda")
        lse = torch.empty((wl.batch, wl.num_q_heads), device="cuda")
        for _ in range(args.warmup):
            paged.run_partial(wl, rc, q, sl, o, lse, ws)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            a.record()
            paged.run_partial(wl, rc, q, sl, o, lse, ws)
            b.record()
        torch.cuda.synchronize()
        t = float(np.median([a.elapsed_time(b) for a, b in evs]))  # ms
        H = wl.num_q_heads
        pages = int(((rc.local_lens + wl.block_size - 1) // wl.block_size).sum())
        kv = rc.total_local * wl.qk_dim * 2
        call = kv + wl.batch * H * (wl.qk_dim * 2 + wl.v_dim * 4 + 4) + pages * 4
        L = np.asarray(wl.lengths)
        rows.append({
            "band": "%d-%s" % (lo, "inf" if hi > di.MAX_SEQ_LEN else str(hi)),
            "batch": wl.batch, "median_len": int(np.median(L)), "max_len": int(L.max()),
            "rank0_local_tokens": int(rc.total_local), "call_ms": round(t, 4),
            "rank0_kv_gbps": round(kv / (t * 1e-3) / 1e9, 1),
            "roofline_frac": round(call / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "local_tokens_per_s": round(rc.total_local / (t * 1e-3), 1),
        })
        del q, sl, rc, ws, o, lse
        torch.cuda.empty_cache()
    print(json.dumps({
        "metric": "rank-0 local-shard decode-attn KV GB/s by request length band",
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "MLA decode, 64 query heads, 576-dim latent KV (V = first 512), "
                               "pages of 128 tokens, N=8 ranks, interleave I=128; rank 0's partial "
                               "call; per band the synthetic length mix restricted to the band, "
                               "batch sized for ~1.25M rank-0 tokens"},
        "bands": rows,
    }), flush=True)


def _event_ms(fn, steps: int, warmup: int) -> float:
    """Median milliseconds of fn() over `steps` calls, HIP events on the launch stream around
    every call, no synchronisation between the calls."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def _event_ms_calls(fns, steps: int, warmup: int) -> np.ndarray:
    """Milliseconds of each call of fns (called in turn, `steps` rounds), HIP events on the
    launch stream around every call, no synchronisation between the calls; [steps, len(fns)]."""
    import torch
    for _ in range(warmup):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
           for _ in range(steps)]
    for row in evs:
        for (a, b), fn in zip(row, fns):
            a.record()
            fn()
            b.record()
    torch.cuda.synchronize()
    return np.array([[a.elapsed_time(b) for a, b in row] for row in evs])


def hbm_read_probe(steps: int, warmup: int, nbytes: int = 4 << 30):
    """Attainable HBM read bandwidth on this device: the harness's streaming-read probe
    (plain 16-byte loads) over a buffer larger than the caches, best of two grid sizes."""
    import torch
    import dcp_inputs as di
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    best = None
    for blocks in (256, 512, 1024):
        t = _event_ms(lambda: di.hbm_read_probe(buf, sink, blocks), max(steps, 5), max(warmup, 1))
        gbps = nbytes / (t * 1e-3) / 1e9
        if best is None or gbps > best[0]:
            best = (gbps, blocks, t)
    del buf, sink
    torch.cuda.empty_cache()
    return {"gbps": round(best[0], 1), "bytes": nbytes, "blocks": best[1], "ms": round(best[2], 4),
            "kind": "streaming read, non-temporal 16-byte vector loads, 8 in flight per thread, "
                    "256-thread work-groups, buffer zero-filled"}


def run_next(args):
    """Multi-token queries, KV append and the per-rank merge steps on the long-context
    MLA batch (the workload of --workload, default B=128, 64 heads, N=8, I=128)."""
    import torch
    import dcp_inputs as di
    import decode_attention_sequence_paged_amd as dcp
    from dcp_inputs import paged

    dcp.lib()
    torch.cuda.set_device(0)
    wl = di.WORKLOADS[args.workload or "mla_long_b128"]
    if wl.kind != "mla":
        raise SystemExit("--next runs on an MLA workload")
    N, B, H, Dqk, Dv, bs = wl.dcp_size, wl.batch, wl.num_q_heads, wl.qk_dim, wl.v_dim, wl.block_size
    desc = paged.desc_for(wl)
    sl = torch.tensor(np.asarray(wl.lengths, dtype=np.int32), device="cuda")
    out = {"metric": "steps next to the hot path: multi-token partial, KV append, per-rank merge steps",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": describe(wl)}}

    # multi-token decode queries, q_len = 1, 2, 4: the calls of ranks 0..3 in turn, events
    # around every call; median over the calls of all four ranks
    NR = min(N, 4)
    rcs = [paged.build_rank_cache(wl, r) for r in range(NR)]
    pages = np.mean([int(((rc.local_lens + bs - 1) // bs).sum()) for rc in rcs])
    local = float(np.mean([rc.total_local for rc in rcs]))
    kv = local * Dqk * 2
    mtp = []
    for q_len in (1, 2, 4):
        qw = di.Workload(**dict(wl.__dict__, batch=B * q_len, lengths=tuple(wl.lengths) * q_len))
        q = paged.device_query(qw).view(B, q_len, H, Dqk)
        ws = paged.workspace_for(wl, 0, q_len=q_len)
        o = torch.empty((B, q_len, H, Dv), device="cuda")
        lse = torch.empty((B, q_len, H), device="cuda")
        fns = [(lambda rc=rc: dcp.dcp_decode_partial_mtp(desc, q, rc.k_cache, None, rc.block_table, sl,
                                                         rc.rank, N, wl.interleave, ws, o, lse))
               for rc in rcs]
        ms = _event_ms_calls(fns, args.steps, args.warmup)
        t = float(np.median(ms))
        call = kv + B * q_len * H * (Dqk * 2 + Dv * 4 + 4) + pages * 4
        mtp.append({"q_len": q_len, "score_rows_per_request": q_len * H,
                    "call_ms_median": round(t, 4), "call_ms_p10": round(float(np.percentile(ms, 10)), 4),
                    "call_ms_p90": round(float(np.percentile(ms, 90)), 4),
                    "kv_gbps": round(kv / (t * 1e-3) / 1e9, 1),
                    "roofline_frac": round(call / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                    "flops_per_s": round(2.0 * q_len * H * (Dqk + Dv) * local / (t * 1e-3), 1)})
        del q, ws, o, lse, fns
    out["multi_token_queries"] = {"ranks": NR, "rows": mtp}
    del rcs
    torch.cuda.empty_cache()

    # GQA multi-token queries (passes of up to four query tokens on as many MFMA column blocks)
    gw = di.WORKLOADS["gqa_b32"]
    gdesc = paged.desc_for(gw)
    gsl = torch.tensor(np.asarray(gw.lengths, dtype=np.int32), device="cuda")
    grcs = [paged.build_rank_cache(gw, r) for r in range(gw.dcp_size)]
    GB, GH = gw.batch, gw.num_q_heads
    gkv = float(np.mean([grc.total_local for grc in grcs])) * gw.num_kv_heads * (gw.qk_dim + gw.v_dim) * 2
    gmtp = []
    for q_len in (1, 2, 4):
        qw = di.Workload(**dict(gw.__dict__, batch=GB * q_len, lengths=tuple(gw.lengths) * q_len))
        q = paged.device_query(qw).view(GB, q_len, GH, gw.qk_dim)
        ws = paged.workspace_for(gw, 0, q_len=q_len)
        o = torch.empty((GB, q_len, GH, gw.v_dim), device="cuda")
        lse = torch.empty((GB, q_len, GH), device="cuda")
        fns = [(lambda grc=grc: dcp.dcp_decode_partial_mtp(gdesc, q, grc.k_cache, grc.v_cache,
                                                           grc.block_table, gsl, grc.rank, gw.dcp_size,
                                                           gw.interleave, ws, o, lse))
               for grc in grcs]
        t = float(np.median(_event_ms_calls(fns, args.steps, args.warmup)))
        passes = q_len // 4 + (q_len % 4) // 2 + q_len % 2  # of 4, 2 and 1 query tokens
        gmtp.append({"q_len": q_len, "passes": passes, "call_ms_median": round(t, 4),
                     "kv_gbps": round(gkv * passes / (t * 1e-3) / 1e9, 1),
                     "ms_per_query_token": round(t / q_len, 4)})
        del q, ws, o, lse, fns
    out["gqa_multi_token_queries"] = {"workload": describe(gw), "ranks": gw.dcp_size, "rows": gmtp}
    del grcs
    torch.cuda.empty_cache()

    # KV append: every rank's call; only the owner of position L-1 writes a request's row
    caches = [paged.build_rank_cache(wl, r) for r in range(N)]
    new_k = torch.randn((B, Dqk), device="cuda").to(torch.bfloat16)

    def append_all():
        for r in range(N):
            dcp.dcp_append_kv(desc, new_k, None, caches[r].k_cache, None, caches[r].block_table, sl,
                              r, N, wl.interleave)
    t = _event_ms(append_all, args.steps, args.warmup)
    out["kv_append"] = {"calls": N, "step_ms": round(t, 4), "call_us": round(1e3 * t / N, 2),
                        "rows_written": B, "bytes_written": B * Dqk * 2}
    del caches
    torch.cuda.empty_cache()

    # the merge as per-rank steps, on partials of the real shape
    o_all = torch.randn((N, B, H, Dv), device="cuda")
    l_all = torch.randn((N, B, H), device="cuda") + 10.0
    o = torch.empty((B, H, Dv), device="cuda")
    lse = torch.empty((B, H), device="cuda")
    gl = torch.empty((B, H), device="cuda")
    row = B * H * Dv * 4
    t_fused = _event_ms(lambda: dcp.dcp_merge(o_all, l_all, o, lse), args.steps, args.warmup)
    t_lse = _event_ms(lambda: dcp.dcp_merge_lse(l_all, gl), args.steps, args.warmup)
    steps = {"fused_merge_ms": round(t_fused, 4),
             "fused_merge_gbps": round((N + 1) * B * H * (Dv + 1) * 4 / (t_fused * 1e-3) / 1e9, 1),
             "merge_lse_ms": round(t_lse, 4)}
    for name, dt, esz in (("fp32", torch.float32, 4), ("bf16", torch.bfloat16, 2)):
        scaled = torch.empty((N, B, H, Dv), dtype=dt, device="cuda")
        sl_out = torch.empty((B, H // N, Dv), device="cuda")
        t_res = _event_ms(lambda: dcp.dcp_rescale_partial(o_all[0], l_all[0], gl, scaled[0]),
                          args.steps, args.warmup)
        t_sum = _event_ms(lambda: dcp.dcp_sum_head_slice(scaled, 0, sl_out), args.steps, args.warmup)
        steps["rescale_%s_ms" % name] = round(t_res, 4)
        steps["rescale_%s_gbps" % name] = round((row + B * H * 8 + B * H * Dv * esz) / (t_res * 1e-3) / 1e9, 1)
        steps["sum_head_slice_%s_ms" % name] = round(t_sum, 4)
        steps["sum_head_slice_%s_gbps" % name] = round(
            (N * B * (H // N) * Dv * esz + B * (H // N) * Dv * 4) / (t_sum * 1e-3) / 1e9, 1)
        steps["per_rank_%s_ms" % name] = round(t_lse + t_res + t_sum, 4)
        del scaled, sl_out
    out["merge_steps"] = steps
    print(json.dumps(out), flush=True)


class Group:
    """Every rank's page pool of one workload, resident in HBM, and the buffers of a
    step: the N ranks' partial calls (one after another on this GPU) and the N-way merge."""

    def __init__(self, wl, partitions: int = 0):
        import torch
        import decode_attention_sequence_paged_amd as dcp
        from dcp_inputs import paged
        self.wl, self.partitions, self.dcp, self.paged = wl, partitions, dcp, paged
        N, B, H = wl.dcp_size, wl.batch, wl.num_q_heads
        self.q = paged.device_query(wl)
        self.sl = torch.tensor(np.asarray(wl.lengths, dtype=np.int32), device="cuda")
        self.ranks = [paged.build_rank_cache(wl, r) for r in range(N)]
        self.ws = paged.workspace_for(wl, partitions)
        self.o_all = torch.empty((N, B, H, wl.v_dim), device="cuda")
        self.l_all = torch.empty((N, B, H), device="cuda")
        self.o = torch.empty((B, H, wl.v_dim), device="cuda")
        self.lse = torch.empty((B, H), device="cuda")
        torch.cuda.synchronize()
        Dqk, Dv = wl.qk_dim, wl.v_dim
        # KV bytes per local token: MLA one 576-dim latent row serving as K and V; GQA a K
        # and a V row per KV head.
        row = Dqk * 2 if wl.kind == "mla" else wl.num_kv_heads * (Dqk + Dv) * 2
        self.local = np.array([rc.total_local for rc in self.ranks], dtype=np.float64)
        pages = np.array([int(((rc.local_lens + wl.block_size - 1) // wl.block_size).sum())
                          for rc in self.ranks])
        self.kv_bytes = self.local * row
        # compulsory bytes of one partial call: KV rows once, q, O_r, LSE_r, block-table entries
        self.call_bytes = self.kv_bytes + B * H * (Dqk * 2 + Dv * 4 + 4) + pages * 4
        self.merge_bytes = (N + 1) * B * H * (Dv + 1) * 4
        self.flops = 2.0 * H * (Dqk + Dv) * self.local

    def step(self, evs=None):
        """One step; with evs, a pair of HIP events (on the launch stream) around each of the
        N partial calls and the merge."""
        N = self.wl.dcp_size
        for r in range(N):
            if evs is not None:
                evs[r][0].record()
            self.paged.run_partial(self.wl, self.ranks[r], self.q, self.sl, self.o_all[r], self.l_all[r],
                                   self.ws, self.partitions)
            if evs is not None:
                evs[r][1].record()
        if evs is not None:
            evs[N][0].record()
        self.dcp.dcp_merge(self.o_all, self.l_all, self.o, self.lse)
        if evs is not None:
            evs[N][1].record()

    def events(self, steps):
        import torch
        return [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(self.wl.dcp_size + 1)] for _ in range(steps)]

    def timed(self, steps: int, warmup: int, flush=None):
        """Warm-up, then `steps` steps with events around every call, bracketed by
        synchronize; no synchronisation between the steps.  With `flush` (a >= 1 GiB device
        buffer), each step is preceded by a write of the whole buffer, outside the events
        (the wall time then includes the flushes).  Returns (wall seconds, per-call ms
        [steps, N + 1])."""
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = self.events(steps)
        t0 = time.perf_counter()
        for s in range(steps):
            if flush is not None:
                flush.zero_()
            self.step(evs[s])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, np.array([[a.elapsed_time(b) for a, b in e] for e in evs])

    def summary(self, wall: float, per_call: np.ndarray) -> dict:
        """Figures of one timed pass (call durations: median / p10 / p90 over the steps,
        and the mean the roofline uses)."""
        N, steps = self.wl.dcp_size, per_call.shape[0]
        calls = per_call[:, :N]
        t_rank_mean = calls.mean(axis=0)
        t_merge = float(per_call[:, N].mean())
        ms_per_step = wall * 1e3 / steps
        achieved = float(self.call_bytes.mean() / (t_rank_mean.mean() * 1e-3) / 1e9)
        pct = lambda a, q: round(float(np.percentile(a, q)), 4)
        step_event_ms = float(per_call.sum(axis=1).mean())
        return {
            "ms_per_step": round(ms_per_step, 4),
            "kv_gbps": round(float(self.kv_bytes.sum() / (ms_per_step * 1e-3) / 1e9), 2),
            "step_event_ms": round(step_event_ms, 4),
            "rank_call_ms_median": [pct(calls[:, r], 50) for r in range(N)],
            "rank_call_ms_p10": [pct(calls[:, r], 10) for r in range(N)],
            "rank_call_ms_p90": [pct(calls[:, r], 90) for r in range(N)],
            "rank_call_ms_mean": [round(float(x), 4) for x in t_rank_mean],
            "call_ms_median_all_ranks": pct(calls, 50),
            "call_ms_p10_all_ranks": pct(calls, 10),
            "call_ms_p90_all_ranks": pct(calls, 90),
            "merge_ms_median": pct(per_call[:, N], 50),
            "merge_ms_mean": round(t_merge, 4),
            "merge_frac": round(t_merge / step_event_ms, 4),
            "merge_gbps": round(self.merge_bytes / (t_merge * 1e-3) / 1e9, 1),
            "call_achieved_gbps": round(achieved, 2),
            "call_frac": round(achieved / HBM_PEAK_GBPS, 4),
            "rank0_kv_gbps_median": round(float(self.kv_bytes[0] / (np.median(calls[:, 0]) * 1e-3) / 1e9), 2),
            "mfma_pct_bf16_peak": round(100.0 * float(self.flops.mean() / (t_rank_mean.mean() * 1e-3))
                                        / (MFMA_BF16_PEAK_TFLOPS * 1e12), 2),
        }

    def free(self):
        import torch
        del self.ranks, self.q, self.ws, self.o_all, self.l_all, self.o, self.lse
        torch.cuda.empty_cache()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


def single_thread_tiny_oracle():
    """The float64 oracle on one host thread: every rank's partials of the tiny MLA batch
    (B=2, 16 heads, lengths 1000 and 3000, N=2, I=1), math only."""
    import dcp_inputs as di
    import oracle
    from threadpoolctl import threadpool_limits
    wl = di.WORKLOADS["mla_tiny"]
    t_math, tokens = 0.0, 0
    with threadpool_limits(limits=1):
        for _ in range(5):
            for r in range(wl.dcp_size):
                for b in range(wl.batch):
                    toks = oracle.rank_tokens(int(wl.lengths[b]), wl.dcp_size, wl.interleave, r)
                    q, K, V = oracle.request_inputs(wl, b, toks)
                    t0 = time.perf_counter()
                    oracle.attention(q, K, V, wl.softmax_scale)
                    t_math += time.perf_counter() - t0
                    tokens += toks.size
    return {"workload": "mla_tiny (B=2, 16 heads, N=2, I=1), every rank's partials, 5 repetitions",
            "threads": 1, "seconds": round(t_math, 4), "tokens_per_s": round(tokens / t_math, 1),
            "gbps": round(tokens * wl.qk_dim * 2 / t_math / 1e9, 4)}


PER_CONFIG = ("gqa_b32", "mla_long_b128", "mla_1m")


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the N ranks of the DCP group are emulated one after "
              "another on a single device, so --gpus %d is not supported." % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    if args.bands:
        run_bands(args)
        return
    if args.next:
        run_next(args)
        return

    import torch
    import dcp_inputs as di
    import decode_attention_sequence_paged_amd as dcp

    dcp.lib()
    torch.cuda.set_device(0)
    wl = di.WORKLOADS[args.workload or "mla_c512"]
    N = wl.dcp_size
    print("bench: building %s" % wl.name, file=sys.stderr, flush=True)
    g = Group(wl, args.partitions)

    if args.copy_probe_bytes:
        src = torch.empty(args.copy_probe_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # timed region: exactly K steps bracketed by synchronize, HIP events around every call
    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
    wall, per_call = g.timed(args.steps, args.warmup)
    warm = g.summary(wall, per_call)
    # the same steps with a 1 GiB scratch write before each (caches flushed: cold)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    wall_c, per_call_c = g.timed(args.steps, 1, flush=flush)
    cold = g.summary(wall_c, per_call_c)
    del flush
    ms_per_step = warm["ms_per_step"]
    t_rank = np.array(warm["rank_call_ms_mean"])
    achieved = warm["call_achieved_gbps"]
    value = float(g.kv_bytes.sum() / (ms_per_step * 1e-3) / 1e9)
    kernel_desc = ("dcp_decode_partial: %s partial kernel%s, mean over the %d ranks' calls"
                   % (wl.kind, "" if single_kernel_call(wl) else " + split_reduce_kernel", N))
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": describe(wl),
            "global_batch": wl.batch,
            "seq_len": int(np.median(wl.lengths)),
            "parallelism": "dcp%d emulated on 1 GPU" % N,
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "steps_per_s": round(1e3 / ms_per_step, 3),
        "decode_tokens_per_s": round(wl.batch * 1e3 / ms_per_step, 1),
        "steps_per_s_per_rank_equiv": round(1e3 / (t_rank[0] + warm["merge_ms_mean"] / N), 3),
        "rank0_kv_gbps": warm["rank0_kv_gbps_median"],
        "rank0_pct_hbm_peak": round(100.0 * warm["rank0_kv_gbps_median"] / HBM_PEAK_GBPS, 2),
        "rank0_local_kv_tokens_per_s": round(g.local[0] / (warm["rank_call_ms_median"][0] * 1e-3), 1),
        "merge_frac": warm["merge_frac"],
        "mfma_pct_bf16_peak": warm["mfma_pct_bf16_peak"],
        "timing": {"timed_region": warm, "cold_1GiB_flush_before_each_step": cold,
                   "note": "events around every call inside the timed region, no synchronisation "
                           "between steps; call times median/p10/p90 over the steps"},
        "roofline": {
            "bound": "hbm",
            "kernel": kernel_desc,
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(wl.name),
            "bytes_per_launch": round(float(g.call_bytes.mean())),
            "launch_ms": round(float(t_rank.mean()), 4),
            "cold_frac": cold["call_frac"],
        },
    }
    g.free()
    del g
    torch.cuda.empty_cache()

    # the other workloads: every rank's call and the merge, same protocol (timed region)
    per_config = {}
    if not args.no_per_config:
        for name in PER_CONFIG:
            if name == wl.name:
                continue
            print("bench: per-config %s" % name, file=sys.stderr, flush=True)
            cw = di.WORKLOADS[name]
            cg = Group(cw)
            wall_x, pc_x = cg.timed(args.steps, args.warmup)
            sx = cg.summary(wall_x, pc_x)
            per_config[name] = {
                "workload": describe(cw),
                "calls": "partial kernel%s" % ("" if single_kernel_call(cw) else " + split_reduce_kernel"),
                "call_frac": sx["call_frac"], "call_ms_median": sx["call_ms_median_all_ranks"],
                "call_ms_p10": sx["call_ms_p10_all_ranks"], "call_ms_p90": sx["call_ms_p90_all_ranks"],
                "rank_call_ms_median": sx["rank_call_ms_median"],
                "ms_per_step": sx["ms_per_step"], "kv_gbps": sx["kv_gbps"],
                "pct_hbm_peak": round(100.0 * sx["kv_gbps"] / HBM_PEAK_GBPS, 2),
                "merge_frac": sx["merge_frac"], "mfma_pct_bf16_peak": sx["mfma_pct_bf16_peak"],
                "steps_per_s": round(1e3 / sx["ms_per_step"], 3),
            }
            cg.free()
            del cg
            torch.cuda.empty_cache()
    out["per_config"] = per_config

    probe = hbm_read_probe(args.steps, args.warmup)
    out["hbm_read_probe"] = probe
    out["roofline"]["frac_of_probe"] = round(achieved / probe["gbps"], 4)
    if not args.no_cpu_baseline:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
        out["cpu_baseline"]["cpu_model"] = cpu_model()
        out["cpu_baseline"]["single_thread_tiny"] = single_thread_tiny_oracle()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
