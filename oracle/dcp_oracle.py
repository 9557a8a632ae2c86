"""Float64 CPU oracle for decode attention over a sequence-sharded paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports or calls this
module; only the test suite, the smoke check and the benchmark's CPU-baseline leg
do.  It shares no code with the HIP library: it sees the *logical*, unsharded
inputs (regenerated from the seeded generator) and enumerates shard ownership
itself.

Sources (the vLLM blog "Efficient Decode Context Parallelism with vLLM for Long
Context Workloads"):

* Sec. 4 ("What is DCP?"): each GPU holds the KV cache of a subset of the token
  positions of every request; Sec. 2.2: each GPU stores only 1/N of a request's KV.
* Sec. 4.1 ("Decode Context Parallelism Process"): every GPU attends the full
  single-token query against its local KV slice, producing a partial output and a
  log-sum-exp; the LSE values reweight and merge the partials (the rescaling online
  softmax also uses) into the exact full-context result.
* Sec. 5.3 (MLA backend): one latent KV vector shared by all query heads.
* Sec. 5.4 (GQA backend): each KV head is shared by (broadcast to) its group of
  query heads.

Readings taken where the pages are silent (each is listed in the design notes):

* token ``t`` belongs to rank ``(t // I) % N`` (interleave size ``I``); the
  contiguous example of Sec. 4 (tokens 0-50K on GPU 0, 50K-100K on GPU 1, ...) is
  the case ``I = L / N``;
* LSE is the natural log of ``sum_t exp(scale * q . k_t)``; partial outputs are
  normalised (``O_r = sum_t p_t v_t / sum_t p_t``);
* MLA uses the weight-absorbed form: the query lives in the 576-dim latent space,
  K is the whole latent row and V its first ``v_dim`` entries;
* GQA query head ``h`` reads KV head ``h // (H / Hkv)``;
* a single decode query attends every cached token (no mask);
* multi-token decode queries (speculative decoding / multi-token prediction, blog
  Sec. 6): the ``q_len`` queries are the request's last ``q_len`` positions, whose
  K/V are already in the cache (``seq_lens`` counts them); query ``i`` attends the
  positions ``<= L - q_len + i`` (causal by global position), so the last query sees
  every token and ``q_len = 1`` is the single-token decode;
* an empty token set gives ``O = 0`` and ``LSE = -inf``, the merge's neutral element.
"""
from __future__ import annotations

import numpy as np

import dcp_inputs as di

NEG_INF = float("-inf")


# ----------------------------------------------------------------------------- shard ownership

def owner_rank(t, N: int, I: int):
    """Rank that holds global token position ``t``: runs of ``I`` tokens dealt round-robin."""
    return (np.asarray(t) // I) % N


def rank_tokens(L: int, N: int, I: int, rank: int) -> np.ndarray:
    """Ascending global positions of the tokens of a length-``L`` request held by ``rank``."""
    t = np.arange(L, dtype=np.int64)
    return t[owner_rank(t, N, I) == rank]


def rank_length(L: int, N: int, I: int, rank: int) -> int:
    """How many of the ``L`` tokens ``rank`` holds (by enumeration)."""
    return int(rank_tokens(L, N, I, rank).size)


# ----------------------------------------------------------------------------- attention

def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Single-token softmax attention for one request, in float64.

    q: [H, Dqk]; K: [L, Hkv, Dqk]; V: [L, Hkv, Dv] (any real dtype, widened to float64).
    Returns (O [H, Dv], LSE [H]) with LSE = ln sum_t exp(scale * q.k_t).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    H = q.shape[0]
    L, Hkv = K.shape[0], K.shape[1]
    Dv = V.shape[2]
    if H % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = H // Hkv
    O = np.zeros((H, Dv), dtype=np.float64)
    LSE = np.full(H, NEG_INF, dtype=np.float64)
    if L == 0:
        return O, LSE
    for g in range(Hkv):
        heads = slice(g * G, (g + 1) * G)
        s = scale * (K[:, g, :] @ q[heads].T)          # [L, G] logits
        m = s.max(axis=0)                                # [G]
        e = np.exp(s - m)                                # [L, G]
        l = e.sum(axis=0)                                # [G]
        O[heads] = (e.T @ V[:, g, :]) / l[:, None]
        LSE[heads] = m + np.log(l)
    return O, LSE


def merge(O_parts, LSE_parts):
    """LSE-weighted merge of partial results over disjoint token sets.

    O_parts: [P, ..., Dv]; LSE_parts: [P, ...].  Parts with LSE = -inf (empty
    token sets) carry no weight; if every part is empty the result is O = 0,
    LSE = -inf.
    """
    O_parts = np.asarray(O_parts, dtype=np.float64)
    LSE_parts = np.asarray(LSE_parts, dtype=np.float64)
    m = LSE_parts.max(axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(LSE_parts - m_safe)                       # exp(-inf) = 0 for empty parts
    total = w.sum(axis=0)
    lse = np.where(empty, NEG_INF, m_safe + np.log(np.where(empty, 1.0, total)))
    scale = np.where(empty, 0.0, 1.0 / np.where(empty, 1.0, total))
    O = (w[..., None] * O_parts).sum(axis=0) * scale[..., None]
    return O, lse


# ----------------------------------------------------------------------------- per-request inputs

def _query(wl, b: int, seed: int) -> np.ndarray:
    H = wl.num_q_heads
    rows = np.arange(b * H, (b + 1) * H, dtype=np.uint64)
    return di.host_rows_f64(rows, wl.qk_dim, seed, di.STREAM_Q)


def mla_inputs(wl, b: int, tokens, seed=None):
    """(q [H,576], K [T,1,576], V [T,1,v_dim]) in float64 for request ``b`` at global ``tokens``."""
    seed = wl.seed if seed is None else seed
    q = _query(wl, b, seed)
    lat = di.host_latent_f64(b, tokens, wl.qk_dim, seed)
    return q, lat[:, None, :], lat[:, None, :wl.v_dim]


def gqa_inputs(wl, b: int, tokens, seed=None):
    """(q [H,D], K [T,Hkv,D], V [T,Hkv,D]) in float64 for request ``b`` at global ``tokens``."""
    seed = wl.seed if seed is None else seed
    q = _query(wl, b, seed)
    K = di.host_gqa_kv_f64(b, tokens, wl.num_kv_heads, wl.qk_dim, seed, di.STREAM_K)
    V = di.host_gqa_kv_f64(b, tokens, wl.num_kv_heads, wl.v_dim, seed, di.STREAM_V)
    return q, K, V


def request_inputs(wl, b: int, tokens, seed=None):
    return (mla_inputs if wl.kind == "mla" else gqa_inputs)(wl, b, tokens, seed)


def rank_partial(wl, b: int, rank: int, seed=None):
    """(O_r, LSE_r) of request ``b`` on ``rank``: attention over the tokens it holds."""
    L = int(wl.lengths[b])
    toks = rank_tokens(L, wl.dcp_size, wl.interleave, rank)
    q, K, V = request_inputs(wl, b, toks, seed)
    return attention(q, K, V, wl.softmax_scale)


def full_attention(wl, b: int, seed=None):
    """(O, LSE) of request ``b`` over its whole context, no sharding."""
    L = int(wl.lengths[b])
    q, K, V = request_inputs(wl, b, np.arange(L, dtype=np.int64), seed)
    return attention(q, K, V, wl.softmax_scale)


# ----------------------------------------------------------------------------- multi-token queries

def causal_limits(L: int, q_len: int) -> np.ndarray:
    """Last global position each of the ``q_len`` queries of a length-``L`` request sees."""
    return L - q_len + np.arange(q_len, dtype=np.int64)


def causal_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, positions, limits, scale: float):
    """Multi-token decode attention in float64: query ``i`` attends the rows whose global
    position is at most ``limits[i]``.

    q: [Q, H, Dqk]; K: [T, Hkv, Dqk]; V: [T, Hkv, Dv]; positions: [T]; limits: [Q].
    Returns (O [Q, H, Dv], LSE [Q, H]); a query that sees no row gets O = 0, LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    Q, H = q.shape[0], q.shape[1]
    Dv = np.asarray(V).shape[2]
    O = np.zeros((Q, H, Dv), dtype=np.float64)
    LSE = np.full((Q, H), NEG_INF, dtype=np.float64)
    for i in range(Q):
        sel = positions <= limits[i]
        O[i], LSE[i] = attention(q[i], np.asarray(K)[sel], np.asarray(V)[sel], scale)
    return O, LSE


def mtp_query(wl, b: int, q_len: int, seed=None) -> np.ndarray:
    """The ``q_len`` query rows of request ``b``: [q_len, H, Dqk]; query ``i`` is logical
    query row ``b * q_len + i`` (so ``q_len = 1`` gives the single-token query)."""
    seed = wl.seed if seed is None else seed
    return np.stack([_query(wl, b * q_len + i, seed) for i in range(q_len)])


def mtp_rank_partial(wl, b: int, rank: int, q_len: int, seed=None):
    """(O_r [Q,H,Dv], LSE_r [Q,H]) of request ``b``'s ``q_len`` queries on ``rank``."""
    seed = wl.seed if seed is None else seed
    L = int(wl.lengths[b])
    toks = rank_tokens(L, wl.dcp_size, wl.interleave, rank)
    _, K, V = request_inputs(wl, b, toks, seed)
    return causal_attention(mtp_query(wl, b, q_len, seed), K, V, toks, causal_limits(L, q_len),
                            wl.softmax_scale)


def mtp_full_attention(wl, b: int, q_len: int, seed=None):
    """(O [Q,H,Dv], LSE [Q,H]) of request ``b``'s ``q_len`` queries over its whole context."""
    seed = wl.seed if seed is None else seed
    L = int(wl.lengths[b])
    toks = np.arange(L, dtype=np.int64)
    _, K, V = request_inputs(wl, b, toks, seed)
    return causal_attention(mtp_query(wl, b, q_len, seed), K, V, toks, causal_limits(L, q_len),
                            wl.softmax_scale)
