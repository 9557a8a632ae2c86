"""dcp_decode_partial_noalloc (the library's static device scratch instead of a caller
workspace) against dcp_decode_partial on the same inputs, through the C ABI: two calls in a
row per kind, the second with a smaller input, each within the parity tolerances of the
workspace call (the kernels are the same, so the results are expected to be identical);
and the rejection of a call whose workspace would not fit the scratch."""
import numpy as np
import pytest
import torch

import dcp_inputs as di
import decode_attention_sequence_paged_amd as dcp

pytestmark = pytest.mark.gpu

TOL_O = 5e-3
TOL_LSE = 1e-3


def _paged():
    from dcp_inputs import paged
    return paged


def _both(wl, rank):
    pg = _paged()
    rc = pg.build_rank_cache(wl, rank)
    q = pg.device_query(wl)
    sl = torch.tensor(np.asarray(wl.lengths, dtype=np.int32), device="cuda")
    shape_o = (wl.batch, wl.num_q_heads, wl.v_dim)
    o1 = torch.full(shape_o, float("nan"), device="cuda")
    l1 = torch.full(shape_o[:2], float("nan"), device="cuda")
    o2 = torch.full(shape_o, float("nan"), device="cuda")
    l2 = torch.full(shape_o[:2], float("nan"), device="cuda")
    pg.run_partial(wl, rc, q, sl, o1, l1, pg.workspace_for(wl))
    dcp.dcp_decode_partial_noalloc(pg.desc_for(wl), q, rc.k_cache, rc.v_cache, rc.block_table, sl, rank,
                                   wl.dcp_size, wl.interleave, o2, l2)
    torch.cuda.synchronize()
    return o1.cpu().numpy(), l1.cpu().numpy(), o2.cpu().numpy(), l2.cpu().numpy()


def _compare(wl, rank):
    o1, l1, o2, l2 = _both(wl, rank)
    assert np.array_equal(np.isneginf(l1), np.isneginf(l2)), wl.name
    fin = np.isfinite(l1)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(l2[fin])), wl.name
    do = float(np.abs(o1 - o2).max())
    dl = float(np.abs(l1[fin] - l2[fin]).max()) if fin.any() else 0.0
    print("%s rank %d: max|dO| = %g, max|dLSE| = %g" % (wl.name, rank, do, dl), flush=True)
    assert do <= TOL_O and dl <= TOL_LSE, wl.name


@pytest.mark.parametrize("kind", ["mla", "gqa"])
def test_noalloc_matches_workspace_call_twice(kind):
    if kind == "mla":
        big = di.Workload("na_mla", "mla", 6, 64, 1, 576, 512, 128, 8, 128, 51,
                          (70000, 1, 300000, 5000, 0, 131072))
        small = di.Workload("na_mla_small", "mla", 2, 16, 1, 576, 512, 64, 2, 1, 52, (900, 4001))
    else:
        big = di.Workload("na_gqa", "gqa", 8, 64, 4, 128, 128, 16, 4, 1, 53,
                          (20000, 4096, 1, 0, 32768, 777, 9000, 12345))
        small = di.Workload("na_gqa_small", "gqa", 3, 32, 8, 128, 128, 32, 2, 3, 54, (1000, 37, 2))
    _compare(big, 0)
    _compare(small, 1)


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    pg = _paged()
    wl = di.Workload("na_big", "mla", 2, 64, 1, 576, 512, 64, 2, 1, 55, (100, 200))
    rc = pg.build_rank_cache(wl, 0)
    q = pg.device_query(wl)
    sl = torch.tensor(np.asarray(wl.lengths, dtype=np.int32), device="cuda")
    o = torch.empty((2, 64, 512), device="cuda")
    lse = torch.empty((2, 64), device="cuda")
    # 4096 partitions of 64 heads need 1 GiB of split pieces, more than the 72 MiB scratch
    assert dcp.dcp_decode_workspace_size(pg.desc_for(wl), 2, 4096) > (72 << 20)
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_decode_partial_noalloc(pg.desc_for(wl), q, rc.k_cache, None, rc.block_table, sl, 0, 2, 1,
                                       o, lse, num_partitions=4096)
    assert e.value.status == dcp.DCP_ERROR_WORKSPACE
