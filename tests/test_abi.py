"""C-ABI library: it loads, exports every declared entry point, and its host-side
shard map and argument validation behave (no GPU needed: nothing here launches)."""
import os
import re

import numpy as np
import pytest

import decode_attention_sequence_paged_amd as dcp
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "dcp.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(dcp_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = dcp.lib()
    names = _declared()
    assert "dcp_decode_partial" in names and "dcp_merge" in names and "dcp_shard_map" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dcp.EXPORTED)


def test_status_strings():
    assert dcp.status_string(0) == "DCP_SUCCESS"
    assert dcp.status_string(3) == "DCP_ERROR_WORKSPACE"
    assert dcp.status_string(99) == "DCP_ERROR_UNKNOWN"


@pytest.mark.parametrize("N,I", [(1, 1), (2, 1), (3, 5), (4, 16), (8, 128), (7, 1000), (8, 3)])
def test_shard_map_matches_oracle_enumeration(N, I):
    L = np.array([0, 1, 2, 5, 127, 128, 129, 1000, 4095, 4096, 20000, N * I, N * I + 1, 3 * N * I - 1])
    for r in range(N):
        got, tot, mx = dcp.dcp_shard_map(L, N, I, r)
        ref = [oracle.rank_length(int(x), N, I, r) for x in L]
        assert list(got) == ref
        assert tot == sum(ref) and mx == max(ref)
    # owner / local index / inverse, bit-exact against the oracle's enumeration
    Lmax = int(L.max())
    t = np.arange(Lmax)
    owner, local = dcp.dcp_shard_locate(t, N, I)
    assert np.array_equal(owner, oracle.owner_rank(t, N, I))
    for r in range(N):
        toks = oracle.rank_tokens(Lmax, N, I, r)
        assert np.array_equal(local[toks], np.arange(toks.size))       # dense ascending order
        assert np.array_equal(dcp.dcp_shard_global(np.arange(toks.size), N, I, r), toks)


def test_shard_map_pages_example():
    # the pages' 200K-token request on 4 GPUs in 50K runs
    got, _, _ = dcp.dcp_shard_map([200000], 4, 50000, 0)
    assert got[0] == 50000
    owner, local = dcp.dcp_shard_locate([0, 49999, 50000, 199999], 4, 50000)
    assert list(owner) == [0, 0, 1, 3] and list(local) == [0, 49999, 0, 49999]
    # 1M tokens, N = 8, I = 128: 131072 per rank
    for r in range(8):
        assert dcp.dcp_shard_map([1 << 20], 8, 128, r)[0][0] == 131072


def test_host_argument_errors():
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_shard_map([10], 0, 1, 0)
    assert e.value.status == dcp.DCP_ERROR_INVALID_VALUE
    for args in [(2, 1, 2), (2, 1, -1), (2, 0, 0)]:
        with pytest.raises(dcp.DcpError):
            dcp.dcp_shard_map([10], *args)
    with pytest.raises(dcp.DcpError):
        dcp.dcp_shard_map([-1], 2, 1, 0)
    with pytest.raises(dcp.DcpError):
        dcp.dcp_shard_locate([-3], 2, 1)


def test_workspace_size_and_desc_validation():
    mla = dcp.attn_desc(dcp.DCP_KV_MLA_LATENT, 64, 1, 576, 512, 128, 576 ** -0.5)
    n = dcp.dcp_decode_workspace_size(mla, 128, 256)
    # prefixes 2 (B+1) int64, 2P x H LSE, 2P x H x 512 O (each 256-byte aligned) + header
    assert n >= 256 + 8 * 2 * 129 + 4 * 2 * 256 * 64 * 513
    assert dcp.dcp_decode_workspace_size(mla, 128, 0) > 0
    bad = [
        dcp.attn_desc(dcp.DCP_KV_MLA_LATENT, 64, 2, 576, 512, 128, 0.1),   # MLA has one KV head
        dcp.attn_desc(dcp.DCP_KV_MLA_LATENT, 64, 1, 512, 512, 128, 0.1),   # unsupported dims
        dcp.attn_desc(dcp.DCP_KV_MLA_LATENT, 1024, 1, 576, 512, 128, 0.1),  # too many heads
        dcp.attn_desc(dcp.DCP_KV_MLA_LATENT, 64, 1, 576, 512, 48, 0.1),    # page not a tile multiple
        dcp.attn_desc(dcp.DCP_KV_GQA, 64, 3, 128, 128, 16, 0.1),           # H % Hkv != 0
        dcp.attn_desc(dcp.DCP_KV_GQA, 64, 2, 128, 128, 16, 0.1),           # group of 32 > 16
        dcp.attn_desc(dcp.DCP_KV_GQA, 64, 4, 128, 128, 8, 0.1),            # page of 8 tokens
        dcp.attn_desc(7, 64, 4, 128, 128, 16, 0.1),
        dcp.attn_desc(dcp.DCP_KV_GQA, 64, 4, 128, 128, 16, float("nan")),
    ]
    for d in bad:
        assert dcp.dcp_decode_workspace_size(d, 4, 8) == 0
    gqa = dcp.attn_desc(dcp.DCP_KV_GQA, 64, 4, 128, 128, 16, 128 ** -0.5)
    assert dcp.dcp_decode_workspace_size(gqa, 32, 64) > 0


def test_partial_rejects_bad_arguments_before_launching():
    import ctypes
    lib = dcp.lib()
    mla = dcp.attn_desc(dcp.DCP_KV_MLA_LATENT, 64, 1, 576, 512, 128, 0.05)
    fake = 1 << 20  # never dereferenced: validation fails first
    def call(desc=mla, q=fake, k=fake, v=0, nb=10, bt=fake, mb=4, sl=fake, B=2, rank=0, N=2, I=1,
             parts=8, ws=fake * 2, wsb=1 << 30, o=fake, lse=fake):
        return lib.dcp_decode_partial(ctypes.byref(desc), q, k, v, nb, bt, mb, sl, B, rank, N, I, parts,
                                      ws, wsb, o, lse, 0)
    assert call(rank=2) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(N=0) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(I=0) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(v=fake) == dcp.DCP_ERROR_INVALID_VALUE       # MLA takes no V cache
    assert call(q=0) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(q=fake + 2) == dcp.DCP_ERROR_INVALID_VALUE   # misaligned
    assert call(nb=0) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(wsb=100) == dcp.DCP_ERROR_WORKSPACE
    assert call(ws=0) == dcp.DCP_ERROR_WORKSPACE
    assert call(B=0) == dcp.DCP_SUCCESS                       # empty batch: nothing to do
    gqa = dcp.attn_desc(dcp.DCP_KV_GQA, 64, 4, 128, 128, 16, 0.05)
    assert call(desc=gqa, v=0) == dcp.DCP_ERROR_INVALID_VALUE  # GQA needs a V cache
    assert lib.dcp_merge(fake, fake, 0, 2, 2, 512, fake, fake, 0) == dcp.DCP_ERROR_INVALID_VALUE
    assert lib.dcp_merge(fake, fake, 2, 2, 2, 510, fake, fake, 0) == dcp.DCP_ERROR_INVALID_VALUE
    assert lib.dcp_merge(fake, fake, 2, 0, 2, 512, fake, fake, 0) == dcp.DCP_SUCCESS


def test_append_rejects_bad_arguments_before_launching():
    import ctypes
    lib = dcp.lib()
    mla = dcp.attn_desc(dcp.DCP_KV_MLA_LATENT, 64, 1, 576, 512, 128, 0.05)
    gqa = dcp.attn_desc(dcp.DCP_KV_GQA, 64, 4, 128, 128, 16, 0.05)
    fake = 1 << 20  # never dereferenced: validation fails first
    def call(desc=mla, nk=fake, nv=0, k=fake, v=0, nb=10, bt=fake, mb=4, sl=fake, B=2, rank=0, N=2, I=1):
        return lib.dcp_append_kv(ctypes.byref(desc), nk, nv, k, v, nb, bt, mb, sl, B, rank, N, I, 0)
    assert call(rank=2) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(rank=-1) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(N=0) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(I=0) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(nv=fake) == dcp.DCP_ERROR_INVALID_VALUE        # MLA has no separate V row
    assert call(v=fake) == dcp.DCP_ERROR_INVALID_VALUE         # ... nor a V cache
    assert call(nk=0) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(k=fake + 8) == dcp.DCP_ERROR_INVALID_VALUE     # misaligned
    assert call(nb=0) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(mb=0) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(B=-1) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(B=0) == dcp.DCP_SUCCESS                         # empty batch: nothing to do
    assert call(desc=gqa) == dcp.DCP_ERROR_INVALID_VALUE        # GQA needs V row and cache
    assert call(desc=gqa, nv=fake) == dcp.DCP_ERROR_INVALID_VALUE
    bad = dcp.attn_desc(dcp.DCP_KV_MLA_LATENT, 64, 1, 576, 512, 48, 0.05)
    assert call(desc=bad) == dcp.DCP_ERROR_NOT_SUPPORTED


def test_merge_steps_reject_bad_arguments_before_launching():
    lib = dcp.lib()
    fake = 1 << 20
    F32, BF16 = dcp.DCP_DTYPE_F32, dcp.DCP_DTYPE_BF16
    assert lib.dcp_merge_lse(fake, 0, 2, 4, fake, 0) == dcp.DCP_ERROR_INVALID_VALUE
    assert lib.dcp_merge_lse(0, 2, 2, 4, fake, 0) == dcp.DCP_ERROR_INVALID_VALUE
    assert lib.dcp_merge_lse(fake, 2, 0, 4, fake, 0) == dcp.DCP_SUCCESS
    assert lib.dcp_rescale_partial(fake, fake, fake, 2, 4, 510, F32, fake, 0) == dcp.DCP_ERROR_INVALID_VALUE
    assert lib.dcp_rescale_partial(fake, fake, fake, 2, 4, 512, 7, fake, 0) == dcp.DCP_ERROR_INVALID_VALUE
    assert lib.dcp_rescale_partial(fake, fake, fake, 2, 4, 512, F32, fake + 8, 0) == dcp.DCP_ERROR_INVALID_VALUE
    assert lib.dcp_rescale_partial(fake, 0, fake, 2, 4, 512, BF16, fake, 0) == dcp.DCP_ERROR_INVALID_VALUE
    assert lib.dcp_rescale_partial(fake, fake, fake, 0, 4, 512, BF16, fake, 0) == dcp.DCP_SUCCESS
    assert lib.dcp_sum_head_slice(fake, F32, 3, 2, 64, 512, 0, fake, 0) == dcp.DCP_ERROR_INVALID_VALUE  # 64 % 3
    assert lib.dcp_sum_head_slice(fake, F32, 4, 2, 64, 512, 4, fake, 0) == dcp.DCP_ERROR_INVALID_VALUE  # rank
    assert lib.dcp_sum_head_slice(fake, 5, 4, 2, 64, 512, 0, fake, 0) == dcp.DCP_ERROR_INVALID_VALUE
    assert lib.dcp_sum_head_slice(fake + 4, BF16, 4, 2, 64, 512, 0, fake, 0) == dcp.DCP_ERROR_INVALID_VALUE
    assert lib.dcp_sum_head_slice(fake, BF16, 4, 0, 64, 512, 0, fake, 0) == dcp.DCP_SUCCESS


def test_mtp_entry_point_validation():
    import ctypes
    lib = dcp.lib()
    mla = dcp.attn_desc(dcp.DCP_KV_MLA_LATENT, 64, 1, 576, 512, 128, 0.05)
    gqa = dcp.attn_desc(dcp.DCP_KV_GQA, 64, 4, 128, 128, 16, 0.05)
    assert dcp.dcp_decode_workspace_size_mtp(mla, 1, 4, 8) == dcp.dcp_decode_workspace_size(mla, 4, 8)
    assert dcp.dcp_decode_workspace_size_mtp(mla, 4, 4, 8) > dcp.dcp_decode_workspace_size(mla, 4, 8)
    assert dcp.dcp_decode_workspace_size_mtp(mla, 0, 4, 8) == 0
    assert dcp.dcp_decode_workspace_size_mtp(mla, 9, 4, 8) == 0      # 9 x 64 rows > 512
    # GQA: passes of up to four query tokens, so the pieces of one four-token pass
    one = dcp.dcp_decode_workspace_size(gqa, 4, 8)
    size = lambda q_len: dcp.dcp_decode_workspace_size_mtp(gqa, q_len, 4, 8)
    assert size(1) == one > 0
    assert size(64) == size(4) > size(2) > one
    assert dcp.dcp_decode_workspace_size_mtp(gqa, 65, 4, 8) == 0
    fake = 1 << 20
    def call(desc=mla, q_len=2, B=2, rank=0):
        return lib.dcp_decode_partial_mtp(ctypes.byref(desc), q_len, fake, fake, 0, 10, fake, 4, fake, B,
                                          rank, 2, 1, 8, fake * 2, 1 << 30, fake, fake, 0)
    assert call(q_len=0) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(q_len=9) == dcp.DCP_ERROR_NOT_SUPPORTED
    assert call(desc=gqa) == dcp.DCP_ERROR_INVALID_VALUE           # GQA needs its V pool
    assert call(desc=gqa, q_len=65) == dcp.DCP_ERROR_NOT_SUPPORTED
    assert call(rank=2) == dcp.DCP_ERROR_INVALID_VALUE
    assert call(B=0) == dcp.DCP_SUCCESS
