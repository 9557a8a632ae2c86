"""Python binding of libdcp (include/dcp.h): argument marshalling only.

Every function has the name of the C entry point it calls and the same argument
order; host arrays are numpy arrays, device buffers are torch CUDA tensors (used
only as storage).  Each call raises ``DcpError`` when the C call returns a status
other than DCP_SUCCESS.  Loading fails loudly when the library is not built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from .build import LIB_PATH

DCP_SUCCESS = 0
DCP_ERROR_INVALID_VALUE = 1
DCP_ERROR_NOT_SUPPORTED = 2
DCP_ERROR_WORKSPACE = 3
DCP_ERROR_HIP = 4

DCP_KV_MLA_LATENT = 0
DCP_KV_GQA = 1
DCP_DTYPE_F32 = 0
DCP_DTYPE_BF16 = 1
DCP_DEVERR_PAGE_ID = 1
DCP_DEVERR_TABLE_SHORT = 2
DCP_DEVERR_NEG_LENGTH = 4


def _torch():
    import torch
    return torch


class DcpError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s" % (fn, status_string(status)))


class AttnDesc(ctypes.Structure):
    """dcp_attn_desc_t."""
    _fields_ = [("kind", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("qk_dim", ctypes.c_int32),
                ("v_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


_lib: Optional[ctypes.CDLL] = None

_i32, _i64, _sz, _vp, _f = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_SIGS = {
    "dcp_status_string": (ctypes.c_char_p, [_i32]),
    "dcp_shard_map": (_i32, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "dcp_shard_locate": (_i32, [_vp, _i64, _i32, _i32, _vp, _vp]),
    "dcp_shard_global": (_i32, [_vp, _i64, _i32, _i32, _i32, _vp]),
    "dcp_shard_map_device": (_i32, [_vp, _i32, _i32, _i32, _i32, _vp, _vp]),
    "dcp_local_block_table": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _vp]),
    "dcp_decode_workspace_size": (_sz, [ctypes.POINTER(AttnDesc), _i32, _i32]),
    "dcp_decode_partial": (_i32, [ctypes.POINTER(AttnDesc), _vp, _vp, _vp, _i64, _vp, _i32, _vp,
                                  _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp, _vp, _vp]),
    "dcp_merge": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "dcp_append_kv": (_i32, [ctypes.POINTER(AttnDesc), _vp, _vp, _vp, _vp, _i64, _vp, _i32, _vp,
                             _i32, _i32, _i32, _i32, _vp]),
    "dcp_merge_lse": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp]),
    "dcp_decode_workspace_size_mtp": (_sz, [ctypes.POINTER(AttnDesc), _i32, _i32, _i32]),
    "dcp_decode_partial_mtp": (_i32, [ctypes.POINTER(AttnDesc), _i32, _vp, _vp, _vp, _i64, _vp, _i32,
                                      _vp, _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp, _vp, _vp]),
    "dcp_rescale_partial": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp]),
    "dcp_sum_head_slice": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "dcp_decode_partial_noalloc": (_i32, [ctypes.POINTER(AttnDesc), _vp, _vp, _vp, _i64, _vp, _i32, _vp,
                                          _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "dcp_workspace_init": (_i32, [_vp, _sz, _vp]),
    "dcp_workspace_errors": (_i32, [_vp, _sz, _vp, _i32, _vp]),
}
EXPORTED = tuple(_SIGS)


def lib() -> ctypes.CDLL:
    """The loaded libdcp.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libdcp.so is not built (expected at %s); run __graft_entry__.build()"
                               % LIB_PATH)
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().dcp_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != DCP_SUCCESS:
        raise DcpError(fn, status)


def _host(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def _dptr(t) -> int:
    """Device pointer of a CUDA tensor (0 for None)."""
    if t is None:
        return 0
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("expected a contiguous CUDA tensor")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return int(stream)


def attn_desc(kind: int, num_q_heads: int, num_kv_heads: int, qk_dim: int, v_dim: int,
              block_size: int, softmax_scale: float) -> AttnDesc:
    return AttnDesc(kind, num_q_heads, num_kv_heads, qk_dim, v_dim, block_size, softmax_scale)


# ----------------------------------------------------------------------------- shard map (host)

def dcp_shard_map(seq_lens, num_ranks: int, interleave: int, rank: int):
    """Returns (local_lens int32 [B], total_local, max_local)."""
    sl, p = _host(seq_lens, np.int32)
    out = np.empty(sl.size, dtype=np.int32)
    tot, mx = ctypes.c_int64(0), ctypes.c_int32(0)
    _check("dcp_shard_map", lib().dcp_shard_map(p, sl.size, num_ranks, interleave, rank,
                                                out.ctypes.data, ctypes.addressof(tot),
                                                ctypes.addressof(mx)))
    return out, tot.value, mx.value


def dcp_shard_locate(positions, num_ranks: int, interleave: int):
    """Returns (owner int32 [n], local_index int64 [n])."""
    pos, p = _host(positions, np.int64)
    owner = np.empty(pos.size, dtype=np.int32)
    local = np.empty(pos.size, dtype=np.int64)
    _check("dcp_shard_locate", lib().dcp_shard_locate(p, pos.size, num_ranks, interleave,
                                                      owner.ctypes.data, local.ctypes.data))
    return owner, local


def dcp_shard_global(local_index, num_ranks: int, interleave: int, rank: int):
    li, p = _host(local_index, np.int64)
    out = np.empty(li.size, dtype=np.int64)
    _check("dcp_shard_global", lib().dcp_shard_global(p, li.size, num_ranks, interleave, rank,
                                                      out.ctypes.data))
    return out


# ----------------------------------------------------------------------------- device calls

def dcp_shard_map_device(seq_lens, num_ranks: int, interleave: int, rank: int, local_lens,
                         stream=None) -> None:
    _check("dcp_shard_map_device", lib().dcp_shard_map_device(
        _dptr(seq_lens), seq_lens.numel(), num_ranks, interleave, rank, _dptr(local_lens),
        _stream(stream)))


def dcp_local_block_table(global_block_table, num_ranks: int, interleave: int, block_size: int,
                          rank: int, local_block_table, stream=None) -> None:
    B, mg = global_block_table.shape
    ml = local_block_table.shape[1]
    _check("dcp_local_block_table", lib().dcp_local_block_table(
        _dptr(global_block_table), B, mg, num_ranks, interleave, block_size, rank,
        _dptr(local_block_table), ml, _stream(stream)))


def dcp_workspace_init(workspace, stream=None) -> None:
    """Zero a partial-attention workspace (once, after allocation)."""
    _check("dcp_workspace_init", lib().dcp_workspace_init(
        _dptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def dcp_workspace_errors(workspace, clear: bool = False, stream=None) -> int:
    """The workspace's device error word (DCP_DEVERR_* bits); synchronises the stream."""
    bits = ctypes.c_uint32(0)
    _check("dcp_workspace_errors", lib().dcp_workspace_errors(
        _dptr(workspace), workspace.numel() * workspace.element_size(), ctypes.addressof(bits),
        1 if clear else 0, _stream(stream)))
    return int(bits.value)


def dcp_decode_workspace_size(desc: AttnDesc, batch: int, num_partitions: int = 0) -> int:
    return int(lib().dcp_decode_workspace_size(ctypes.byref(desc), batch, num_partitions))


def dcp_decode_partial(desc: AttnDesc, q, k_cache, v_cache, block_table, seq_lens, rank: int,
                       num_ranks: int, interleave: int, workspace, out_o, out_lse,
                       num_partitions: int = 0, stream=None) -> None:
    """One rank's partial attention; shapes as in include/dcp.h."""
    batch = q.shape[0]
    _check("dcp_decode_partial", lib().dcp_decode_partial(
        ctypes.byref(desc), _dptr(q), _dptr(k_cache), _dptr(v_cache), k_cache.shape[0],
        _dptr(block_table), block_table.shape[1], _dptr(seq_lens), batch, rank, num_ranks,
        interleave, num_partitions, _dptr(workspace), workspace.numel() * workspace.element_size(),
        _dptr(out_o), _dptr(out_lse), _stream(stream)))


def dcp_decode_partial_noalloc(desc: AttnDesc, q, k_cache, v_cache, block_table, seq_lens, rank: int,
                               num_ranks: int, interleave: int, out_o, out_lse, num_partitions: int = 0,
                               stream=None) -> None:
    """dcp_decode_partial with the library's static device scratch instead of a workspace."""
    batch = q.shape[0]
    _check("dcp_decode_partial_noalloc", lib().dcp_decode_partial_noalloc(
        ctypes.byref(desc), _dptr(q), _dptr(k_cache), _dptr(v_cache), k_cache.shape[0],
        _dptr(block_table), block_table.shape[1], _dptr(seq_lens), batch, rank, num_ranks,
        interleave, num_partitions, _dptr(out_o), _dptr(out_lse), _stream(stream)))


def dcp_append_kv(desc: AttnDesc, new_k, new_v, k_cache, v_cache, block_table, seq_lens,
                  rank: int, num_ranks: int, interleave: int, stream=None) -> None:
    """Write each request's newest token row into the owning rank's page (see
    include/dcp.h); a rank's call touches only the requests it owns."""
    _check("dcp_append_kv", lib().dcp_append_kv(
        ctypes.byref(desc), _dptr(new_k), _dptr(new_v), _dptr(k_cache), _dptr(v_cache),
        k_cache.shape[0], _dptr(block_table), block_table.shape[1], _dptr(seq_lens),
        new_k.shape[0], rank, num_ranks, interleave, _stream(stream)))


def dcp_merge_lse(lse_parts, out_lse, stream=None) -> None:
    """Global LSE [B,H] from the gathered per-rank LSEs [N,B,H]."""
    N, B, H = lse_parts.shape
    _check("dcp_merge_lse", lib().dcp_merge_lse(_dptr(lse_parts), N, B, H, _dptr(out_lse),
                                                _stream(stream)))


def dcp_rescale_partial(o_r, lse_r, lse, out, stream=None) -> None:
    """out = exp(lse_r - lse) * o_r; out is float32 or bfloat16 [B,H,Dv]."""
    B, H, Dv = o_r.shape
    dt = DCP_DTYPE_BF16 if out.dtype == _torch().bfloat16 else DCP_DTYPE_F32
    _check("dcp_rescale_partial", lib().dcp_rescale_partial(
        _dptr(o_r), _dptr(lse_r), _dptr(lse), B, H, Dv, dt, _dptr(out), _stream(stream)))


def dcp_sum_head_slice(scaled_parts, rank: int, out, stream=None) -> None:
    """Rank `rank`'s head slice of the sum over the stacked scaled partials
    [N,B,H,Dv] (float32 or bfloat16); out float32 [B, H/N, Dv]."""
    N, B, H, Dv = scaled_parts.shape
    dt = DCP_DTYPE_BF16 if scaled_parts.dtype == _torch().bfloat16 else DCP_DTYPE_F32
    _check("dcp_sum_head_slice", lib().dcp_sum_head_slice(
        _dptr(scaled_parts), dt, N, B, H, Dv, rank, _dptr(out), _stream(stream)))


def dcp_decode_workspace_size_mtp(desc: AttnDesc, q_len: int, batch: int, num_partitions: int = 0) -> int:
    return int(lib().dcp_decode_workspace_size_mtp(ctypes.byref(desc), q_len, batch, num_partitions))


def dcp_decode_partial_mtp(desc: AttnDesc, q, k_cache, v_cache, block_table, seq_lens, rank: int,
                           num_ranks: int, interleave: int, workspace, out_o, out_lse,
                           num_partitions: int = 0, stream=None) -> None:
    """One rank's partial attention for q_len query tokens per request, causal by global
    position: q [B, q_len, H, qk_dim]; out_o [B, q_len, H, v_dim]; out_lse [B, q_len, H]."""
    batch, q_len = q.shape[0], q.shape[1]
    _check("dcp_decode_partial_mtp", lib().dcp_decode_partial_mtp(
        ctypes.byref(desc), q_len, _dptr(q), _dptr(k_cache), _dptr(v_cache), k_cache.shape[0],
        _dptr(block_table), block_table.shape[1], _dptr(seq_lens), batch, rank, num_ranks,
        interleave, num_partitions, _dptr(workspace), workspace.numel() * workspace.element_size(),
        _dptr(out_o), _dptr(out_lse), _stream(stream)))


def dcp_merge(o_parts, lse_parts, out_o, out_lse, stream=None) -> None:
    """N-way LSE merge: o_parts [N,B,H,Dv], lse_parts [N,B,H] -> out_o [B,H,Dv], out_lse [B,H]."""
    N, B, H, Dv = o_parts.shape
    _check("dcp_merge", lib().dcp_merge(_dptr(o_parts), _dptr(lse_parts), N, B, H, Dv, _dptr(out_o),
                                        _dptr(out_lse), _stream(stream)))
