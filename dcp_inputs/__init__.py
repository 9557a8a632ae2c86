"""Seeded synthetic inputs for decode attention over a sequence-sharded paged KV cache.

This module is shared by the float64 oracle's tests and by the GPU harness
(tests, bench, smoke).  It holds *no* attention, softmax, shard-ownership or merge
arithmetic: only value generation, request-length sampling, page-id shuffling and
workload shapes.

Value generator
---------------
Every bf16 input element is a pure function of (seed, stream, logical row, column),
so a value never depends on how tokens are sharded or paged:

* splitmix64 (Steele, Lea & Flood, "Fast Splittable Pseudorandom Number Generators",
  OOPSLA 2014) evaluated at a counter: ``draw(n) = mix64(key + (n + 1) * GOLDEN)``
  with ``key = mix64((seed * 65536 + stream) * GOLDEN)``.
* An element with counter ``c = row * 1024 + col`` takes draws ``3c, 3c+1, 3c+2``;
  their twelve 16-bit fields ``u_i`` give an Irwin-Hall(12) approximately standard
  normal value ``z = (sum(u_i) - 393210) / 65536`` (mean 0, variance
  ``(65536**2 - 1) / 65536**2``, ``|z| <= 6``), exact in fp32.
* ``z`` is rounded to bf16 with round-to-nearest-even.

The device implementation (``csrc/synth_fill.hip``) follows the same definition and
is checked bit-for-bit against this one.

Logical row ids (``ROW_T_BITS`` leaves room for 2**21 tokens per request):

* query:            ``row = b * H + h``                       (stream ``STREAM_Q``)
* MLA latent cache: ``row = b * 2**21 + t``                  (stream ``STREAM_K``)
* GQA K / V cache:  ``row = (b * 2**21 + t) * Hkv + g``       (``STREAM_K`` / ``STREAM_V``)

where ``t`` is the request's *global* token position.
"""
from __future__ import annotations

import ctypes
import math
import os
import statistics
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

GOLDEN = 0x9E3779B97F4A7C15
MIX_C1 = 0xBF58476D1CE4E5B9
MIX_C2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

STREAM_Q = 0
STREAM_K = 1
STREAM_V = 2
STREAM_LENGTHS = 3
STREAM_PAGES = 4

ROW_T_BITS = 21
MAX_COLS = 1024
IH12_MEAN = 393210  # 12 * (65535 / 2)

_U64 = np.uint64


def _mix64_py(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX_C1) & MASK64
    z = ((z ^ (z >> 27)) * MIX_C2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int) -> int:
    """64-bit key of one (seed, stream) pair."""
    return _mix64_py(((seed * 65536 + stream) * GOLDEN) & MASK64)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> _U64(30))) * _U64(MIX_C1)
    z = (z ^ (z >> _U64(27))) * _U64(MIX_C2)
    return z ^ (z >> _U64(31))


def splitmix64_at(key: int, n: np.ndarray) -> np.ndarray:
    """splitmix64 output number ``n`` (0-based) of the stream that starts at ``key``."""
    n = np.asarray(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64_np(_U64(key) + (n + _U64(1)) * _U64(GOLDEN))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = _U64(0x7FFF) + ((b >> _U64(16)) & _U64(1))
    return ((b + bias) >> _U64(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns exactly to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def host_rows_numpy(row_ids, cols: int, seed: int, stream: int,
                    chunk_rows: int = 1 << 14) -> np.ndarray:
    """bf16 bit patterns [len(row_ids), cols] for the given logical rows (pure numpy)."""
    if cols > MAX_COLS:
        raise ValueError("at most %d columns per row" % MAX_COLS)
    row_ids = np.asarray(row_ids, dtype=np.uint64).reshape(-1)
    key = stream_key(seed, stream)
    out = np.empty((row_ids.size, cols), dtype=np.uint16)
    col = np.arange(cols, dtype=np.uint64)
    for s in range(0, row_ids.size, chunk_rows):
        r = row_ids[s:s + chunk_rows]
        c = r[:, None] * _U64(MAX_COLS) + col[None, :]
        acc = np.zeros(c.shape, dtype=np.int64)
        for i in range(3):
            d = splitmix64_at(key, c * _U64(3) + _U64(i))
            for f in range(4):
                acc += ((d >> _U64(16 * f)) & _U64(0xFFFF)).astype(np.int64)
        z = (acc - IH12_MEAN).astype(np.float32) / np.float32(65536.0)
        out[s:s + chunk_rows] = f32_to_bf16_bits(z)
    return out


def census_rows_numpy(row_ids, cols: int) -> np.ndarray:
    """Census rows: element (row, col) is 1.0 when bit ``col`` of ``row`` is set (col < 24)."""
    row_ids = np.asarray(row_ids, dtype=np.uint64).reshape(-1)
    col = np.arange(cols, dtype=np.uint64)
    bit = ((row_ids[:, None] >> np.minimum(col, _U64(63))[None, :]) & _U64(1)).astype(bool)
    bit &= (col < _U64(24))[None, :]
    return np.where(bit, np.uint16(0x3F80), np.uint16(0)).astype(np.uint16)


_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB_PATH = os.path.join(_HERE, "libdcp_synth_host.so")
_host_lib: Optional[ctypes.CDLL] = None


def _host_lib_handle() -> Optional[ctypes.CDLL]:
    global _host_lib
    if _host_lib is None and os.path.exists(HOST_LIB_PATH):
        lib = ctypes.CDLL(HOST_LIB_PATH)
        for fn in (lib.dcp_synth_host_rows, lib.dcp_synth_host_rows_f64):
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64,
                           ctypes.c_int32, ctypes.c_void_p]
        _host_lib = lib
    return _host_lib


def host_rows(row_ids, cols: int, seed: int, stream: int, mode: int = 0) -> np.ndarray:
    """bf16 bit patterns [len(row_ids), cols]; mode 0 = seeded normals, 1 = census bits.

    Uses the compiled host generator when it is built (same definition, much faster),
    else the numpy one.
    """
    if cols > MAX_COLS:
        raise ValueError("at most %d columns per row" % MAX_COLS)
    row_ids = np.ascontiguousarray(np.asarray(row_ids, dtype=np.uint64).reshape(-1))
    lib = _host_lib_handle()
    if lib is None:
        return census_rows_numpy(row_ids, cols) if mode == 1 else \
            host_rows_numpy(row_ids, cols, seed, stream)
    out = np.empty((row_ids.size, cols), dtype=np.uint16)
    if row_ids.size:
        rc = lib.dcp_synth_host_rows(row_ids.ctypes.data, row_ids.size, cols,
                                     stream_key(seed, stream), mode, out.ctypes.data)
        if rc != 0:
            raise RuntimeError("dcp_synth_host_rows failed")
    return out


def host_rows_f64(row_ids, cols: int, seed: int, stream: int, mode: int = 0) -> np.ndarray:
    """The values of host_rows (bf16) widened exactly to float64 [len(row_ids), cols]."""
    if cols > MAX_COLS:
        raise ValueError("at most %d columns per row" % MAX_COLS)
    row_ids = np.ascontiguousarray(np.asarray(row_ids, dtype=np.uint64).reshape(-1))
    lib = _host_lib_handle()
    if lib is None:
        return bf16_bits_to_f64(host_rows(row_ids, cols, seed, stream, mode))
    out = np.empty((row_ids.size, cols), dtype=np.float64)
    if row_ids.size:
        rc = lib.dcp_synth_host_rows_f64(row_ids.ctypes.data, row_ids.size, cols,
                                         stream_key(seed, stream), mode, out.ctypes.data)
        if rc != 0:
            raise RuntimeError("dcp_synth_host_rows_f64 failed")
    return out


# ----------------------------------------------------------------------------- rows

def q_row_ids(batch: int, heads: int) -> np.ndarray:
    return np.arange(batch * heads, dtype=np.uint64)


def latent_row_ids(b: int, tokens) -> np.ndarray:
    t = np.asarray(tokens, dtype=np.uint64)
    return (_U64(b) << _U64(ROW_T_BITS)) + t


def gqa_row_ids(b: int, tokens, num_kv_heads: int, kv_head: int) -> np.ndarray:
    t = np.asarray(tokens, dtype=np.uint64)
    return ((_U64(b) << _U64(ROW_T_BITS)) + t) * _U64(num_kv_heads) + _U64(kv_head)


def host_query(batch: int, heads: int, dim: int, seed: int) -> np.ndarray:
    """bf16 bits [batch, heads, dim]."""
    return host_rows(q_row_ids(batch, heads), dim, seed, STREAM_Q).reshape(batch, heads, dim)


def host_latent(b: int, tokens, dim: int, seed: int) -> np.ndarray:
    """bf16 bits [len(tokens), dim] of request ``b``'s latent rows at global positions ``tokens``."""
    return host_rows(latent_row_ids(b, tokens), dim, seed, STREAM_K)


def host_latent_f64(b: int, tokens, dim: int, seed: int) -> np.ndarray:
    """host_latent's values widened to float64."""
    return host_rows_f64(latent_row_ids(b, tokens), dim, seed, STREAM_K)


def host_gqa_kv_f64(b: int, tokens, num_kv_heads: int, dim: int, seed: int, stream: int) -> np.ndarray:
    """host_gqa_kv's values widened to float64."""
    t = np.asarray(tokens, dtype=np.uint64)
    rows = ((_U64(b) << _U64(ROW_T_BITS)) + t)[:, None] * _U64(num_kv_heads) + \
        np.arange(num_kv_heads, dtype=np.uint64)[None, :]
    return host_rows_f64(rows.reshape(-1), dim, seed, stream).reshape(t.size, num_kv_heads, dim)


def host_gqa_kv(b: int, tokens, num_kv_heads: int, dim: int, seed: int, stream: int) -> np.ndarray:
    """bf16 bits [len(tokens), num_kv_heads, dim] of K (STREAM_K) or V (STREAM_V)."""
    t = np.asarray(tokens, dtype=np.uint64)
    rows = ((_U64(b) << _U64(ROW_T_BITS)) + t)[:, None] * _U64(num_kv_heads) + \
        np.arange(num_kv_heads, dtype=np.uint64)[None, :]
    return host_rows(rows.reshape(-1), dim, seed, stream).reshape(t.size, num_kv_heads, dim)


# ----------------------------------------------------------------------------- lengths

_LN_LO = math.log(65536.0)
_LN_MID = math.log(262144.0)
_LN_HI = math.log(1048576.0)
LOGN_MU = 9.9926
LOGN_SIGMA = 0.7078
MAX_SEQ_LEN = 1 << 20


def bimodal_length_quantile(u: float) -> int:
    """Inverse CDF of the synthetic agentic length mix (see module docs of workloads)."""
    if u < 0.18:
        return int(1024 + (u / 0.18) * (8192 - 1024))
    if u < 0.47:
        return int(8192 + ((u - 0.18) / 0.29) * (65536 - 8192))
    if u < 0.965:
        nd = statistics.NormalDist(LOGN_MU, LOGN_SIGMA)
        a, c = nd.cdf(_LN_LO), nd.cdf(_LN_MID)
        v = (u - 0.47) / 0.495
        x = math.exp(nd.inv_cdf(a + v * (c - a)))
        return int(min(max(x, 65536.0), 262143.0))
    v = (u - 0.965) / 0.035
    return int(min(math.exp(_LN_MID + v * (_LN_HI - _LN_MID)), float(MAX_SEQ_LEN)))


def bimodal_lengths(batch: int, seed: int) -> np.ndarray:
    """Stratified inverse-CDF draw of ``batch`` request lengths, shuffled with ``seed``."""
    u = (np.arange(batch) + 0.5) / batch
    rng = np.random.default_rng([seed, STREAM_LENGTHS])
    u = u[rng.permutation(batch)]
    return np.array([bimodal_length_quantile(float(x)) for x in u], dtype=np.int64)


def _band_u(length: int) -> float:
    """Smallest u (to 1e-12) with bimodal_length_quantile(u) >= length."""
    lo, hi = 0.0, 1.0
    if bimodal_length_quantile(0.0) >= length:
        return 0.0
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if bimodal_length_quantile(mid) >= length:
            hi = mid
        else:
            lo = mid
    return hi


def band_lengths(lo: int, hi: int, batch: int, seed: int) -> np.ndarray:
    """``batch`` lengths of the synthetic mix restricted to [lo, hi): stratified
    inverse-CDF draws over the part of the distribution that falls into the band,
    shuffled with ``seed``."""
    u0, u1 = _band_u(lo), _band_u(hi) if hi <= MAX_SEQ_LEN else 1.0
    u = u0 + (np.arange(batch) + 0.5) / batch * (u1 - u0)
    rng = np.random.default_rng([seed, STREAM_LENGTHS, lo])
    u = u[rng.permutation(batch)]
    L = np.array([bimodal_length_quantile(float(x)) for x in u], dtype=np.int64)
    return np.clip(L, lo, min(hi, MAX_SEQ_LEN + 1) - 1)


# The length bands of the pages' comparison by sequence length (blog Sec. 2.3).
LENGTH_BANDS = ((0, 32768), (32768, 65536), (65536, 131072), (131072, 204800), (204800, MAX_SEQ_LEN + 1))


def band_workload(lo: int, hi: int, local_tokens: int = 1_250_000, seed: int = 3) -> "Workload":
    """The long-context MLA shape (64 heads, pages of 128, N = 8, I = 128) with requests
    from one length band, as many as give rank 0 about ``local_tokens`` tokens."""
    probe = band_lengths(lo, hi, 64, seed)
    batch = int(min(4096, max(1, round(local_tokens * 8 / float(probe.mean())))))
    L = band_lengths(lo, hi, batch, seed)
    name = "mla_band_%dk_%s" % (lo // 1024, "inf" if hi > MAX_SEQ_LEN else "%dk" % (hi // 1024))
    return Workload(name, "mla", batch, 64, 1, 576, 512, 128, 8, 128, seed, tuple(int(x) for x in L))


def uniform_lengths(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, STREAM_LENGTHS])
    return rng.integers(lo, hi + 1, size=batch).astype(np.int64)


def page_permutation(num_pages: int, seed: int, salt: int = 0) -> np.ndarray:
    """A seeded random permutation of physical page ids."""
    rng = np.random.default_rng([seed, STREAM_PAGES, salt])
    return rng.permutation(num_pages).astype(np.int64)


# ----------------------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Workload:
    """Shape of one synthetic decode batch."""
    name: str
    kind: str                 # "mla" or "gqa"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    qk_dim: int
    v_dim: int
    block_size: int
    dcp_size: int             # N
    interleave: int           # I
    seed: int
    lengths: tuple = field(default=())

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.qk_dim)

    def seq_lens(self) -> np.ndarray:
        return np.asarray(self.lengths, dtype=np.int64)


def _make_workloads() -> dict:
    w = {}
    w["mla_tiny"] = Workload("mla_tiny", "mla", 2, 16, 1, 576, 512, 64, 2, 1, 1,
                             (1000, 3000))
    w["gqa_b32"] = Workload("gqa_b32", "gqa", 32, 64, 4, 128, 128, 16, 4, 1, 2,
                            tuple(int(x) for x in uniform_lengths(32, 4096, 32768, 2)))
    w["mla_long_b128"] = Workload("mla_long_b128", "mla", 128, 64, 1, 576, 512, 128, 8, 128, 3,
                                  tuple(int(x) for x in bimodal_lengths(128, 3)))
    w["mla_c512"] = Workload("mla_c512", "mla", 512, 64, 1, 576, 512, 128, 8, 128, 4,
                             tuple(int(x) for x in bimodal_lengths(512, 4)))
    w["mla_1m"] = Workload("mla_1m", "mla", 1, 128, 1, 576, 512, 128, 8, 128, 5, (1 << 20,))
    return w


WORKLOADS = _make_workloads()


# ----------------------------------------------------------------------------- device fill

SYNTH_LIB_PATH = os.path.join(_HERE, "libdcp_synth.so")
_synth_lib: Optional[ctypes.CDLL] = None


def synth_lib() -> ctypes.CDLL:
    """The device-side generator library (built from csrc/synth_fill.hip)."""
    global _synth_lib
    if _synth_lib is None:
        if not os.path.exists(SYNTH_LIB_PATH):
            raise RuntimeError("libdcp_synth.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(SYNTH_LIB_PATH)
        lib.dcp_synth_fill_rows.restype = ctypes.c_int
        lib.dcp_synth_fill_rows.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p]
        lib.dcp_synth_fill_value.restype = ctypes.c_int
        lib.dcp_synth_fill_value.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint16,
                                             ctypes.c_void_p]
        lib.dcp_hbm_read_probe.restype = ctypes.c_int
        lib.dcp_hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_int32, ctypes.c_void_p]
        _synth_lib = lib
    return _synth_lib


def device_fill_rows(dst, dst_rows, row_ids, cols: int, seed: int, stream: int,
                     mode: int = 0, hip_stream: int = 0) -> None:
    """Write generated rows into a device bf16 tensor.

    ``dst`` is a contiguous 16-bit CUDA tensor viewed as rows of ``cols`` elements;
    ``dst_rows`` / ``row_ids`` are int64 CUDA tensors of equal length: element
    ``(dst_rows[i], c)`` receives the generated value of logical ``(row_ids[i], c)``.
    Destination rows outside the tensor are skipped.
    """
    n = int(dst_rows.numel())
    if n == 0:
        return
    assert row_ids.numel() == n and dst.is_contiguous()
    assert dst_rows.dtype == row_ids.dtype and str(row_ids.dtype) == "torch.int64"
    key = stream_key(seed, stream)
    rc = synth_lib().dcp_synth_fill_rows(
        ctypes.c_void_p(dst.data_ptr()), ctypes.c_int64(dst.numel() // cols),
        ctypes.c_void_p(dst_rows.data_ptr()), ctypes.c_void_p(row_ids.data_ptr()),
        ctypes.c_int64(n), ctypes.c_int32(cols), ctypes.c_uint64(key), ctypes.c_int32(mode),
        ctypes.c_void_p(hip_stream))
    if rc != 0:
        raise RuntimeError("dcp_synth_fill_rows failed with code %d" % rc)


BF16_NAN_BITS = 0x7FC0


def device_fill_value(dst, bits: int, hip_stream: int = 0) -> None:
    """Fill a device 16-bit tensor with one bit pattern (e.g. a NaN poison)."""
    rc = synth_lib().dcp_synth_fill_value(ctypes.c_void_p(dst.data_ptr()),
                                          ctypes.c_int64(dst.numel()), ctypes.c_uint16(bits),
                                          ctypes.c_void_p(hip_stream))
    if rc != 0:
        raise RuntimeError("dcp_synth_fill_value failed with code %d" % rc)


def hbm_read_probe(buf, sink, blocks: int, hip_stream: int = 0) -> None:
    """Launch the streaming-read probe over the bytes of the contiguous CUDA tensor
    ``buf`` (a harness measurement; ``sink`` is a CUDA tensor of >= 1024 int32)."""
    nbytes = buf.numel() * buf.element_size()
    assert buf.is_contiguous() and sink.numel() >= 1024
    rc = synth_lib().dcp_hbm_read_probe(ctypes.c_void_p(buf.data_ptr()), ctypes.c_int64(nbytes),
                                        ctypes.c_void_p(sink.data_ptr()), ctypes.c_int32(blocks),
                                        ctypes.c_void_p(hip_stream))
    if rc != 0:
        raise RuntimeError("dcp_hbm_read_probe failed (%d)" % rc)
