"""Pins of the float64 oracle against facts that do not come from the oracle itself.

Each ``check_*`` function takes the implementation under test (attention, merge,
rank-token enumeration) so that ``test_planted_mistakes_are_caught`` can run the
same pins against deliberately broken copies of the oracle and show that every
planted mistake fails at least one pin.

Independent references used here:
* the pages' worked ownership example (tests/golden/contiguous_split_200k_4gpu.txt);
* the pages' statement that each GPU holds 1/N of a request's KV (blog Sec. 2.2);
* the pages' statement that the reweighted merge of the partials is the exact
  full-context result (blog Sec. 4.1): sharded-then-merged must equal unsharded attention;
* torch's CPU ``scaled_dot_product_attention`` and scipy's ``logsumexp`` in float64;
* closed forms (q = 0, constant V, one token, two tokens, dominant logit) and bounds;
* brute force in pure-Python loops on tiny inputs.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import dcp_inputs as di
import oracle
from oracle import dcp_oracle as odc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _rand_case(rng, H=8, Hkv=2, L=37, D=24, Dv=16):
    q = rng.standard_normal((H, D))
    K = rng.standard_normal((L, Hkv, D))
    V = rng.standard_normal((L, Hkv, Dv))
    return q, K, V, 1.0 / math.sqrt(D)


class Impl:
    def __init__(self, attention=oracle.attention, merge=oracle.merge,
                 rank_tokens=oracle.rank_tokens, causal_attention=oracle.causal_attention,
                 causal_limits=oracle.causal_limits, request_inputs=oracle.request_inputs,
                 mtp_query=oracle.mtp_query):
        self.attention = attention
        self.merge = merge
        self.rank_tokens = rank_tokens
        self.causal_attention = causal_attention
        self.causal_limits = causal_limits
        self.request_inputs = request_inputs
        self.mtp_query = mtp_query


# ----------------------------------------------------------------------------- pins

def check_contiguous_example(impl):
    """The pages' 200K-tokens-on-4-GPUs example (blog Sec. 4)."""
    for L, N, I, r, lo, hi in _read_table("contiguous_split_200k_4gpu.txt"):
        toks = impl.rank_tokens(int(L), int(N), int(I), int(r))
        assert toks.size == int(hi) - int(lo)
        assert toks[0] == int(lo) and toks[-1] == int(hi) - 1
        assert np.array_equal(toks, np.arange(int(lo), int(hi)))


def check_one_nth(impl):
    """Each rank holds exactly L/N tokens when L is a multiple of N*I (blog Sec. 2.2)."""
    for L, N, I in [(1 << 20, 8, 128), (4096, 4, 1), (6000, 2, 1000), (960, 8, 3)]:
        for r in range(N):
            assert impl.rank_tokens(L, N, I, r).size == L // N


def check_partition(impl):
    """Shards are disjoint and cover every position; each rank owns whole runs of I."""
    for L, N, I in [(0, 3, 2), (1, 4, 16), (37, 3, 5), (1000, 8, 128), (513, 2, 1), (100, 7, 1000)]:
        parts = [impl.rank_tokens(L, N, I, r) for r in range(N)]
        allt = np.sort(np.concatenate(parts)) if parts else np.array([])
        assert np.array_equal(allt, np.arange(L))
        # lengths differ by at most I and the remainder goes to the lowest ranks
        lens = [p.size for p in parts]
        assert max(lens) - min(lens) <= I if L else True
        assert lens == sorted(lens, reverse=True)


def check_against_torch_sdpa(impl):
    """Attention equals torch's float64 scaled_dot_product_attention (GQA by repeat)."""
    rng = np.random.default_rng(11)
    for (H, Hkv, L, D, Dv) in [(8, 2, 37, 24, 16), (4, 1, 50, 40, 32), (6, 3, 1, 8, 8), (16, 4, 129, 16, 16)]:
        q, K, V, scale = _rand_case(rng, H, Hkv, L, D, Dv)
        O, LSE = impl.attention(q, K, V, scale)
        G = H // Hkv
        qt = torch.from_numpy(q)[:, None, :]                       # [H, 1, D]
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [H, L, D]
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[:, 0, :]
        assert np.allclose(O, ref.numpy(), rtol=1e-12, atol=1e-12)
        for h in range(H):
            s = scale * (K[:, h // G, :] @ q[h])
            assert abs(LSE[h] - scipy.special.logsumexp(s)) < 1e-12 * max(1.0, abs(LSE[h]))


def check_closed_forms(impl):
    rng = np.random.default_rng(12)
    # q = 0: uniform weights -> LSE = ln L, O = mean of V
    q, K, V, scale = _rand_case(rng, 4, 2, 19, 8, 6)
    O, LSE = impl.attention(np.zeros_like(q), K, V, scale)
    assert np.allclose(LSE, math.log(19), atol=1e-13)
    for h in range(4):
        assert np.allclose(O[h], V[:, h // 2, :].mean(axis=0), atol=1e-13)
    # constant V: O = c for any logits
    Vc = np.broadcast_to(np.arange(6, dtype=np.float64), V.shape).copy()
    O, _ = impl.attention(q, K, Vc, scale)
    assert np.allclose(O, np.arange(6.0)[None, :], atol=1e-12)
    # one token: O = v_0, LSE = s_0
    O, LSE = impl.attention(q, K[:1], V[:1], scale)
    for h in range(4):
        assert np.allclose(O[h], V[0, h // 2], atol=1e-14)
        assert abs(LSE[h] - scale * K[0, h // 2] @ q[h]) < 1e-13
    # two tokens: weights are the logistic function of the logit gap
    O, LSE = impl.attention(q, K[:2], V[:2], scale)
    for h in range(4):
        g = h // 2
        s0, s1 = scale * K[0, g] @ q[h], scale * K[1, g] @ q[h]
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        assert np.allclose(O[h], w0 * V[0, g] + (1 - w0) * V[1, g], atol=1e-13)
        assert abs(LSE[h] - np.logaddexp(s0, s1)) < 1e-13
    # a logit that dominates the rest by 40 nats selects its value row
    L = 25
    K = np.zeros((L, 1, 4)); K[7, 0, 0] = 40.0
    q = np.array([[1.0, 0.0, 0.0, 0.0]])
    V = rng.standard_normal((L, 1, 3))
    O, LSE = impl.attention(q, K, V, 1.0)
    assert np.allclose(O[0], V[7, 0], atol=1e-15 * 0 + 1e-15 + 30 * math.exp(-40))
    assert abs(LSE[0] - (40.0 + math.log1p((L - 1) * math.exp(-40.0)))) < 1e-13
    # bounds: max logit <= LSE <= max logit + ln L
    q, K, V, scale = _rand_case(rng, 4, 1, 33, 8, 4)
    _, LSE = impl.attention(q * 5, K, V, scale)
    for h in range(4):
        s = scale * K[:, 0] @ (q[h] * 5)
        assert s.max() - 1e-12 <= LSE[h] <= s.max() + math.log(33) + 1e-12
    # empty token set
    O, LSE = impl.attention(q, K[:0], V[:0], scale)
    assert np.all(O == 0) and np.all(np.isneginf(LSE))


def check_brute_force(impl):
    """Pure-Python loops on tiny inputs."""
    rng = np.random.default_rng(13)
    for (H, Hkv, L, D, Dv) in [(2, 1, 5, 3, 2), (4, 2, 7, 4, 3), (3, 3, 4, 2, 5)]:
        q, K, V, scale = _rand_case(rng, H, Hkv, L, D, Dv)
        O, LSE = impl.attention(q, K, V, scale)
        G = H // Hkv
        for h in range(H):
            g = h // G
            logits = []
            for t in range(L):
                acc = 0.0
                for d in range(D):
                    acc += float(q[h, d]) * float(K[t, g, d])
                logits.append(scale * acc)
            total = sum(math.exp(x) for x in logits)
            assert abs(LSE[h] - math.log(total)) < 1e-12
            for e in range(Dv):
                num = sum(math.exp(logits[t]) * float(V[t, g, e]) for t in range(L))
                assert abs(O[h, e] - num / total) < 1e-12


def check_merge_equals_unsharded(impl):
    """Sharding by position plus the LSE merge equals unsharded attention (blog Sec. 4.1)."""
    rng = np.random.default_rng(14)
    for (L, N, I) in [(1000, 2, 1), (777, 4, 16), (300, 8, 128), (96, 3, 1000), (5000, 8, 3)]:
        q, K, V, scale = _rand_case(rng, 8, 2, L, 16, 12)
        q = q * 3.0  # peaky logits
        O_full, LSE_full = impl.attention(q, K, V, scale)
        parts = [impl.attention(q, K[t], V[t], scale)
                 for t in (impl.rank_tokens(L, N, I, r) for r in range(N))]
        O, LSE = impl.merge([p[0] for p in parts], [p[1] for p in parts])
        assert np.allclose(O, O_full, rtol=1e-12, atol=1e-13)
        assert np.allclose(LSE, LSE_full, rtol=1e-13, atol=1e-13)


def check_merge_identities(impl):
    rng = np.random.default_rng(15)
    q, K, V, scale = _rand_case(rng, 4, 1, 200, 8, 8)
    O1, L1 = impl.attention(q, K, V, scale)
    # N = 1 identity
    O, LSE = impl.merge([O1], [L1])
    assert np.array_equal(O, O1) and np.array_equal(LSE, L1)
    # invariance to N and I, and to the order of the parts
    res = []
    for N, I in [(1, 1), (2, 1), (4, 16), (8, 128), (3, 7), (5, 1000)]:
        parts = [impl.attention(q, K[t], V[t], scale)
                 for t in (impl.rank_tokens(200, N, I, r) for r in range(N))]
        perm = rng.permutation(N)
        O, LSE = impl.merge([parts[i][0] for i in perm], [parts[i][1] for i in perm])
        res.append((O, LSE))
    for O, LSE in res[1:]:
        assert np.allclose(O, res[0][0], rtol=1e-12, atol=1e-13)
        assert np.allclose(LSE, res[0][1], rtol=1e-13, atol=1e-13)
    # an empty part is neutral; all-empty gives O = 0, LSE = -inf
    Oe, Le = impl.attention(q, K[:0], V[:0], scale)
    O, LSE = impl.merge([O1, Oe], [L1, Le])
    assert np.allclose(O, O1, atol=1e-15) and np.allclose(LSE, L1, atol=1e-15)
    O, LSE = impl.merge([Oe, Oe], [Le, Le])
    assert np.all(O == 0) and np.all(np.isneginf(LSE))
    # associativity: merging per-chunk partials then per-rank equals one flat merge
    chunks = [np.arange(0, 50), np.arange(50, 120), np.arange(120, 200)]
    cp = [impl.attention(q, K[c], V[c], scale) for c in chunks]
    Oa, La = impl.merge([cp[0][0], cp[1][0]], [cp[0][1], cp[1][1]])
    O2, L2 = impl.merge([Oa, cp[2][0]], [La, cp[2][1]])
    assert np.allclose(O2, O1, rtol=1e-12, atol=1e-13) and np.allclose(L2, L1, atol=1e-13)
    # a subset of shards merges to attention over the union of their tokens
    t0, t2 = impl.rank_tokens(200, 4, 8, 0), impl.rank_tokens(200, 4, 8, 2)
    p0, p2 = impl.attention(q, K[t0], V[t0], scale), impl.attention(q, K[t2], V[t2], scale)
    O, LSE = impl.merge([p0[0], p2[0]], [p0[1], p2[1]])
    u = np.sort(np.concatenate([t0, t2]))
    Ou, Lu = impl.attention(q, K[u], V[u], scale)
    assert np.allclose(O, Ou, rtol=1e-12, atol=1e-13) and np.allclose(LSE, Lu, atol=1e-13)


def check_large_logits(impl):
    """Logits in the hundreds neither overflow nor lose the merge (online-softmax guard)."""
    rng = np.random.default_rng(16)
    q, K, V, _ = _rand_case(rng, 2, 1, 64, 8, 4)
    scale = 60.0
    O, LSE = impl.attention(q, K, V, scale)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(LSE))
    parts = [impl.attention(q, K[t], V[t], scale)
             for t in (impl.rank_tokens(64, 4, 2, r) for r in range(4))]
    Om, Lm = impl.merge([p[0] for p in parts], [p[1] for p in parts])
    assert np.allclose(Om, O, rtol=1e-10, atol=1e-12) and np.allclose(Lm, LSE, rtol=1e-13)


def _mtp_case(rng, Q=3, H=4, Hkv=2, L=23, D=12, Dv=8):
    q = rng.standard_normal((Q, H, D))
    K = rng.standard_normal((L, Hkv, D))
    V = rng.standard_normal((L, Hkv, Dv))
    return q, K, V, 1.0 / math.sqrt(D)


def check_mtp_single_query_is_decode(impl):
    """One query token: the causal path is the single-token decode over every cached token."""
    rng = np.random.default_rng(11)
    q, K, V, sc = _mtp_case(rng, Q=1)
    L = K.shape[0]
    O, LSE = impl.causal_attention(q, K, V, np.arange(L), impl.causal_limits(L, 1), sc)
    O1, L1 = impl.attention(q[0], K, V, sc)
    assert np.allclose(O[0], O1, rtol=1e-13, atol=1e-14) and np.allclose(LSE[0], L1, atol=1e-13)


def check_mtp_brute_force(impl):
    """Multi-token queries against pure-Python loops: query i (the request's position
    L - Q + i) sums over the tokens at positions <= L - Q + i."""
    rng = np.random.default_rng(12)
    q, K, V, sc = _mtp_case(rng, Q=4, H=4, Hkv=2, L=9, D=5, Dv=3)
    Q, H, L = q.shape[0], q.shape[1], K.shape[0]
    pos = np.arange(L)
    O, LSE = impl.causal_attention(q, K, V, pos, impl.causal_limits(L, Q), sc)
    G = H // K.shape[1]
    for i in range(Q):
        last = L - Q + i
        for h in range(H):
            g = h // G
            s = [sc * sum(q[i, h, d] * K[t, g, d] for d in range(q.shape[2])) for t in range(last + 1)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            assert abs(LSE[i, h] - (m + math.log(tot))) < 1e-12
            for e in range(V.shape[2]):
                ref = sum(w[t] * V[t, g, e] for t in range(last + 1)) / tot
                assert abs(O[i, h, e] - ref) < 1e-12


def check_mtp_closed_form_counts(impl):
    """q = 0 on rank r's tokens: query i sees exactly the rank's tokens among positions
    0..L-Q+i, i.e. rank_length(L-Q+i+1) of them (the per-length formula of the pages'
    1/N split, computed independently of the enumeration); LSE = ln(count) and O is the
    running mean of V over them."""
    N, I, Q = 3, 4, 5
    for L in (1, 3, 11, 12, 13, 40):
        for r in range(N):
            toks = impl.rank_tokens(L, N, I, r)
            T = len(toks)
            V = np.arange(T * 2, dtype=np.float64).reshape(T, 1, 2)
            K = np.ones((T, 1, 3))
            q = np.zeros((Q, 2, 3))
            O, LSE = impl.causal_attention(q, K, V, toks, impl.causal_limits(L, Q), 0.5)
            for i in range(Q):
                n_vis = oracle.rank_length(max(L - Q + i + 1, 0), N, I, r)
                if n_vis == 0:
                    assert np.all(np.isneginf(LSE[i])) and np.all(O[i] == 0)
                    continue
                assert np.allclose(LSE[i], math.log(n_vis), atol=1e-13)
                mean = np.cumsum(V[:, 0, :], axis=0)[n_vis - 1] / n_vis
                assert np.allclose(O[i], mean[None, :], atol=1e-12)


def check_mtp_sharded_merge_equals_unsharded(impl):
    """Blog Sec. 4.1 with causal multi-token queries: the ranks' causal partials merge
    to the unsharded causal attention, for several N and I."""
    rng = np.random.default_rng(13)
    q, K, V, sc = _mtp_case(rng, Q=3, L=29)
    L, Q = K.shape[0], q.shape[0]
    Ou, Lu = impl.causal_attention(q, K, V, np.arange(L), impl.causal_limits(L, Q), sc)
    for N, I in ((2, 1), (3, 4), (4, 2), (5, 16)):
        parts = []
        for r in range(N):
            toks = impl.rank_tokens(L, N, I, r)
            parts.append(impl.causal_attention(q, K[toks], V[toks], toks, impl.causal_limits(L, Q), sc))
        O, LSE = impl.merge([p[0] for p in parts], [p[1] for p in parts])
        assert np.allclose(O, Ou, rtol=1e-12, atol=1e-13) and np.allclose(LSE, Lu, atol=1e-13)


def check_mtp_query_is_a_shorter_request(impl):
    """On every rank, the causal set of query i of a length-L request with Q query tokens
    is the rank's shard of a request of length L - (Q - 1 - i): its causal partial equals
    the single-token partial over that shorter request's tokens on the rank."""
    rng = np.random.default_rng(14)
    q, K, V, sc = _mtp_case(rng, Q=4, H=6, Hkv=3, L=37)
    L, Q = K.shape[0], q.shape[0]
    for N, I in ((1, 1), (3, 2), (4, 5)):
        for r in range(N):
            toks = impl.rank_tokens(L, N, I, r)
            O, LSE = impl.causal_attention(q, K[toks], V[toks], toks, impl.causal_limits(L, Q), sc)
            for i in range(Q):
                short = impl.rank_tokens(L - (Q - 1 - i), N, I, r)
                Os, Ls = impl.attention(q[i], K[short], V[short], sc)
                assert np.allclose(O[i], Os, rtol=1e-13, atol=1e-14), (N, I, r, i)
                assert np.array_equal(np.isneginf(LSE[i]), np.isneginf(Ls))
                fin = np.isfinite(Ls)
                assert np.allclose(LSE[i][fin], Ls[fin], atol=1e-13), (N, I, r, i)


# ----------------------------------------------------------------------------- input readings
#
# Which generated values the oracle takes as q, K and V.  The expectations below are
# built straight from the seeded generator's logical rows (the row-id convention of
# dcp_inputs: query row b*H + h, latent row b*2**21 + t, GQA row (b*2**21 + t)*Hkv + g)
# and the readings of the pages: MLA's K is the whole 576-dim latent row and V its first
# 512 entries (one latent vector shared by every head, blog Sec. 5.3); GQA query head h
# reads KV head h // (H / Hkv) (blog Sec. 5.4), K from the K stream and V from the V
# stream.  Two closed forms pin them: q = 0 gives O = the mean of the V rows, and a
# single cached token gives LSE = scale * q . k over every K dimension.

def _gen(row_ids, cols, seed, stream):
    return di.bf16_bits_to_f64(di.host_rows(np.asarray(row_ids, dtype=np.uint64), cols, seed, stream))


def _latent_row(b, t):
    return b * (1 << 21) + t


def check_mla_input_reading(impl):
    wl = di.Workload("pin_mla", "mla", 3, 4, 1, 576, 512, 64, 3, 2, 41, (37, 5, 80))
    H, sc = wl.num_q_heads, wl.softmax_scale
    for b, toks in ((0, np.array([0, 1, 6, 7, 12, 30, 36])), (1, np.array([2, 3])),
                    (2, np.arange(0, 80, 3))):
        rows = _gen([_latent_row(b, int(t)) for t in toks], 576, wl.seed, di.STREAM_K)
        q, K, V = impl.request_inputs(wl, b, toks)
        O, LSE = impl.attention(np.zeros_like(q), K, V, sc)
        assert np.allclose(LSE, math.log(toks.size), atol=1e-13)
        for h in range(H):
            assert np.allclose(O[h], rows[:, :512].mean(axis=0), rtol=1e-13, atol=1e-14), (b, h)
        qrows = _gen([b * H + h for h in range(H)], 576, wl.seed, di.STREAM_Q)
        for j, t in enumerate(toks[:3]):
            q1, K1, V1 = impl.request_inputs(wl, b, np.array([t]))
            O1, L1 = impl.attention(q1, K1, V1, sc)
            for h in range(H):
                assert abs(L1[h] - sc * float(qrows[h] @ rows[j])) < 1e-12, (b, t, h)
                assert np.array_equal(O1[h], rows[j, :512]), (b, t, h)


def check_gqa_input_reading(impl):
    wl = di.Workload("pin_gqa", "gqa", 2, 8, 4, 128, 128, 16, 2, 1, 42, (30, 7))
    H, Hkv, sc = wl.num_q_heads, wl.num_kv_heads, wl.softmax_scale
    G = H // Hkv
    for b, toks in ((0, np.array([0, 2, 5, 17, 29])), (1, np.array([1, 6]))):
        q, K, V = impl.request_inputs(wl, b, toks)
        O, LSE = impl.attention(np.zeros_like(q), K, V, sc)
        assert np.allclose(LSE, math.log(toks.size), atol=1e-13)
        qrows = _gen([b * H + h for h in range(H)], 128, wl.seed, di.STREAM_Q)
        for h in range(H):
            g = h // G
            ids = [_latent_row(b, int(t)) * Hkv + g for t in toks]
            vrows = _gen(ids, 128, wl.seed, di.STREAM_V)
            krows = _gen(ids, 128, wl.seed, di.STREAM_K)
            assert np.allclose(O[h], vrows.mean(axis=0), rtol=1e-13, atol=1e-14), (b, h)
            q1, K1, V1 = impl.request_inputs(wl, b, toks[:1])
            O1, L1 = impl.attention(q1, K1, V1, sc)
            assert abs(L1[h] - sc * float(qrows[h] @ krows[0])) < 1e-12, (b, h)
            assert np.array_equal(O1[h], vrows[0]), (b, h)


def check_mtp_query_reading(impl):
    """Query token i of request b is the generator's query row (b*q_len + i)*H + h, the
    batch of B*q_len single-token queries viewed as [B, q_len, H]: one cached token
    gives LSE = scale * q . k for every (query token, head)."""
    wl = di.Workload("pin_mtp", "mla", 2, 3, 1, 576, 512, 64, 1, 1, 43, (9, 4))
    H, sc, Q = wl.num_q_heads, wl.softmax_scale, 3
    for b in range(2):
        krow = _gen([_latent_row(b, 0)], 576, wl.seed, di.STREAM_K)
        q = impl.mtp_query(wl, b, Q)
        O, LSE = impl.causal_attention(q, krow[:, None, :], krow[:, None, :512], np.array([0]),
                                       np.zeros(Q, dtype=np.int64), sc)
        for i in range(Q):
            qrows = _gen([(b * Q + i) * H + h for h in range(H)], 576, wl.seed, di.STREAM_Q)
            for h in range(H):
                assert abs(LSE[i, h] - sc * float(qrows[h] @ krow[0])) < 1e-12, (b, i, h)


ALL_CHECKS = [check_contiguous_example, check_one_nth, check_partition, check_against_torch_sdpa,
              check_closed_forms, check_brute_force, check_merge_equals_unsharded,
              check_merge_identities, check_large_logits, check_mtp_single_query_is_decode,
              check_mtp_brute_force, check_mtp_closed_form_counts,
              check_mtp_sharded_merge_equals_unsharded, check_mtp_query_is_a_shorter_request,
              check_mla_input_reading, check_gqa_input_reading, check_mtp_query_reading]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(Impl())


# ----------------------------------------------------------------------------- planted mistakes

def _mut_attention(kind):
    def attn(q, K, V, scale):
        q = np.asarray(q, np.float64); K = np.asarray(K, np.float64); V = np.asarray(V, np.float64)
        H, L, Hkv, Dv = q.shape[0], K.shape[0], K.shape[1], V.shape[2]
        G = H // Hkv
        O = np.zeros((H, Dv)); LSE = np.full(H, -np.inf)
        if L == 0:
            return O, LSE
        for h in range(H):
            g = h % Hkv if kind == "group_mod" else h // G
            sc = 1.0 if kind == "no_scale" else scale
            s = sc * (K[:, g, :] @ q[h])
            if kind == "sign":
                s = -s
            m = s.max()
            e = np.exp(s - m)
            l = e.sum()
            vv = V[:, g, :]
            if kind == "v_offset":
                vv = np.roll(vv, 1, axis=0)
            O[h] = (e @ vv) / (1.0 if kind == "unnormalised" else l)
            LSE[h] = (0.0 if kind == "lse_no_max" else m) + np.log(l)
            if kind == "lse_log2":
                LSE[h] = m + np.log2(l)
            if kind == "drop_last" and L > 1:
                e2 = e[:-1]
                O[h] = (e2 @ vv[:-1]) / e2.sum()
                LSE[h] = m + np.log(e2.sum())
        return O, LSE
    return attn


def _mut_merge(kind):
    def mrg(O_parts, LSE_parts):
        O_parts = np.asarray(O_parts, np.float64); LSE_parts = np.asarray(LSE_parts, np.float64)
        m = LSE_parts.max(axis=0)
        empty = ~np.isfinite(m)
        ms = np.where(empty, 0.0, m)
        w = np.exp(LSE_parts - ms)
        if kind == "uniform_weights":
            w = np.where(np.isfinite(LSE_parts), 1.0, 0.0)
        tot = w.sum(axis=0)
        lse = np.where(empty, -np.inf, ms + np.log(np.where(empty, 1.0, tot)))
        if kind == "lse_max_only":
            lse = m
        sc = 1.0 / np.where(empty, 1.0, tot)
        if kind == "no_renorm":
            sc = np.ones_like(sc)
        O = (w[..., None] * O_parts).sum(axis=0) * sc[..., None]
        if kind == "empty_nan":
            O = (np.exp(LSE_parts - m)[..., None] * O_parts).sum(axis=0) / np.exp(LSE_parts - m).sum(axis=0)[..., None]
            lse = m + np.log(np.exp(LSE_parts - m).sum(axis=0))
        return O, lse
    return mrg


def _mut_tokens(kind):
    def toks(L, N, I, r):
        t = np.arange(L, dtype=np.int64)
        if kind == "mod_first":
            return t[(t % N) // I == r] if I > 1 else t[t % N == r]
        if kind == "block_by_n":
            return t[(t // N) % I == r % max(I, 1)] if I < N else t[(t // I) % N == r]
        if kind == "off_by_one":
            return t[((t + 1) // I) % N == r]
        return t[(t // I) % N == r]
    return toks


def _mut_causal(kind):
    def causal(q, K, V, positions, limits, scale):
        positions = np.asarray(positions)
        if kind == "strict":
            limits = np.asarray(limits) - 1
        if kind == "local_index":  # masks by the rank-local index instead of the position
            positions = np.arange(len(positions))
        if kind == "query_reversed":
            limits = np.asarray(limits)[::-1]
        return oracle.causal_attention(q, K, V, positions, limits, scale)
    return causal


def _mut_limits(kind):
    def lim(L, q_len):
        if kind == "shift":
            return L - q_len + 1 + np.arange(q_len)
        return L - 1 - np.arange(q_len)[::-1] * 0  # every query sees everything
    return lim


def _mut_inputs(kind):
    """Wrong readings of which generated values are q, K and V."""
    def inputs(wl, b, tokens, seed=None):
        seed = wl.seed if seed is None else seed
        t = np.asarray(tokens, dtype=np.int64)
        H = wl.num_q_heads
        qid = [h * wl.batch + b for h in range(H)] if kind == "q_transposed" else \
            [b * H + h for h in range(H)]
        q = _gen(qid, wl.qk_dim, seed, di.STREAM_Q)
        if wl.kind == "mla":
            lat = _gen([_latent_row(b, int(x)) for x in t], wl.qk_dim, seed, di.STREAM_K)
            K = lat.copy()
            V = lat[:, :wl.v_dim]
            if kind == "v_tail":          # V = the last 512 entries (row[64:])
                V = lat[:, -wl.v_dim:]
            if kind == "k_no_rope":       # K = the first 512 entries only
                K[:, wl.v_dim:] = 0.0
            return q, K[:, None, :], V[:, None, :]
        Hkv = wl.num_kv_heads
        g = np.arange(Hkv)
        if kind == "kv_head_reversed":    # query heads read the groups' KV heads in reverse
            g = g[::-1]
        ids = (np.array([_latent_row(b, int(x)) for x in t], dtype=np.int64)[:, None] * Hkv
               + g[None, :]).reshape(-1)
        if kind == "kv_rows_transposed":  # KV head major instead of token major
            ids = ((b * Hkv + np.arange(Hkv))[None, :] * (1 << 21) + t[:, None]).reshape(-1)
        ks, vs = (di.STREAM_V, di.STREAM_K) if kind == "kv_swapped" else (di.STREAM_K, di.STREAM_V)
        K = _gen(ids, wl.qk_dim, seed, ks).reshape(t.size, Hkv, wl.qk_dim)
        V = _gen(ids, wl.v_dim, seed, vs).reshape(t.size, Hkv, wl.v_dim)
        return q, K, V
    return inputs


def _mut_mtp_query(kind):
    def mq(wl, b, q_len, seed=None):
        seed = wl.seed if seed is None else seed
        H = wl.num_q_heads
        rows = [(i * wl.batch + b) * H + h for i in range(q_len) for h in range(H)]
        return _gen(rows, wl.qk_dim, seed, di.STREAM_Q).reshape(q_len, H, wl.qk_dim)
    return mq


MUTANTS = (
    [("attention:" + k, Impl(attention=_mut_attention(k))) for k in
     ["group_mod", "no_scale", "sign", "v_offset", "unnormalised", "lse_no_max", "lse_log2", "drop_last"]]
    + [("merge:" + k, Impl(merge=_mut_merge(k))) for k in
       ["uniform_weights", "lse_max_only", "no_renorm", "empty_nan"]]
    + [("tokens:" + k, Impl(rank_tokens=_mut_tokens(k))) for k in
       ["mod_first", "block_by_n", "off_by_one"]]
    + [("causal:" + k, Impl(causal_attention=_mut_causal(k))) for k in
       ["strict", "local_index", "query_reversed"]]
    + [("limits:" + k, Impl(causal_limits=_mut_limits(k))) for k in ["shift", "no_mask"]]
    + [("inputs:" + k, Impl(request_inputs=_mut_inputs(k))) for k in
       ["q_transposed", "v_tail", "k_no_rope", "kv_head_reversed", "kv_rows_transposed",
        "kv_swapped"]]
    + [("mtp_query:query_major", Impl(mtp_query=_mut_mtp_query("query_major")))]
)


@pytest.mark.parametrize("name,impl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistakes_are_caught(name, impl):
    failed = []
    for check in ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(impl)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, "planted mistake %s passed every pin" % name


def test_dcp_partial_vectors_for_a_workload():
    """Rank partials of a small MLA workload merge to its unsharded attention."""
    import dcp_inputs as di
    wl = di.Workload("mini", "mla", 2, 4, 1, 576, 512, 64, 2, 3, 9, (70, 5))
    for b in range(2):
        parts = [odc.rank_partial(wl, b, r) for r in range(2)]
        O, LSE = oracle.merge([p[0] for p in parts], [p[1] for p in parts])
        Of, Lf = odc.full_attention(wl, b)
        assert np.allclose(O, Of, rtol=1e-12, atol=1e-13) and np.allclose(LSE, Lf, atol=1e-13)
    # request 1 has 5 tokens, I = 3: rank 0 holds {0,1,2}, rank 1 holds {3,4}
    assert list(odc.rank_tokens(5, 2, 3, 0)) == [0, 1, 2]
    assert list(odc.rank_tokens(5, 2, 3, 1)) == [3, 4]
