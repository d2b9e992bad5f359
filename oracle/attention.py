"""Decode and prefill attention through a block table (oracle; test
infrastructure only).

[L] = "Paged Attention: OS-Inspired Memory Management for KV Caches";
[B] = "What is PagedAttention and how does it manage KV cache?".

The pages fix the result exactly: reading keys and values block by block
through the table gives attention identical to the contiguous layout ([L],
"How PagedAttention works", step 4; "Key takeaways": paging is exact;
"Memory sharing across requests": the same numbers, the same outputs). So the
oracle is that definition written out: gather the sequence's tokens through
its table into contiguous arrays, then ordinary softmax attention of the one
new query over all L cached tokens, in fp64.

Readings the pages leave open (they are silent on these points):
  * grouped-query heads: query head h reads KV head h // (Hq / Hkv);
  * the scale is the caller's (1/sqrt(D) in every workload); no bias, cap or
    window;
  * L = 0 gives a zero output;
  * prefill: the pages say only that the prompt's keys and values are stored
    in the blocks the manager hands out ([L], "How PagedAttention works",
    step 1) and that attention reads through the table as if contiguous. The
    plainest reading for a causal decoder: each new token attends to every
    earlier token of its sequence and to itself, and the new tokens are the
    last n of the L stored ones, so a cached prefix (shared prompt blocks,
    [L] "Memory sharing across requests") is attended in full.
"""
from __future__ import annotations

import numpy as np

from .cache import gather


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query [D] over L keys/values [L, D], in fp64.

    scores = scale * K q; weights = exp(scores - max) / sum; out = weights V.
    Subtracting the maximum changes nothing mathematically and keeps exp finite.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    scores = float(scale) * (K @ q)
    w = np.exp(scores - scores.max())
    return (w @ V) / w.sum()


def decode(query, k_pool, v_pool, block_tables, context_lens, scale) -> np.ndarray:
    """Paged decode: out[s, h] = attention of query[s, h] over the first
    context_lens[s] tokens of KV head h // (Hq / Hkv), read through
    block_tables[s]. Returns fp64 [S, Hq, D].
    """
    S, Hq, D = query.shape
    NB, Hkv, B, Dk = k_pool.shape
    if Dk != D or v_pool.shape != k_pool.shape:
        raise ValueError("shape mismatch")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        L = int(context_lens[s])
        if L < 0 or L > block_tables.shape[1] * B:
            raise ValueError("context length outside [0, MB * B]")
        if L == 0:
            continue
        Kc = gather(k_pool, block_tables[s], L, B).astype(np.float64)
        Vc = gather(v_pool, block_tables[s], L, B).astype(np.float64)
        for h in range(Hq):
            g = h // G
            out[s, h] = attend(query[s, h], Kc[g], Vc[g], scale)
    return out


def attend_partial(q, K, V, scale):
    """Unnormalised state of attention over a subset of tokens:
    m = max score, l = sum exp(score - m), acc = sum exp(score - m) V.
    An empty subset gives (-inf, 0, 0)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(V.shape[1])
    scores = float(scale) * (K @ q)
    m = scores.max()
    w = np.exp(scores - m)
    return m, w.sum(), w @ V


def merge_partials(parts):
    """Combine states of disjoint token subsets into the attention output:
    with M = max m_p, out = sum e^(m_p - M) acc_p / sum e^(m_p - M) l_p."""
    ms = np.array([p[0] for p in parts], dtype=np.float64)
    M = ms.max()
    if not np.isfinite(M):
        return np.zeros_like(parts[0][2])
    num = sum(np.exp(m - M) * acc for m, _, acc in parts if np.isfinite(m))
    den = sum(np.exp(m - M) * l for m, l, _ in parts if np.isfinite(m))
    return num / den


def causal_attention(Q, K, V, first_pos: int, scale) -> np.ndarray:
    """Softmax attention of n query rows over L keys/values, causal, in fp64.

    Row i is the token at position first_pos + i and sees keys 0 .. first_pos + i:
    scores = scale * Q K^T with the keys after each row's position removed from
    its softmax, then weights = exp(scores - row max) / row sum and
    out = weights V. Every row must see at least one key (first_pos >= 0).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n, L = Q.shape[0], K.shape[0]
    if first_pos < 0 or first_pos + n > L:
        raise ValueError("rows must sit at positions 0 .. L - 1")
    scores = float(scale) * (Q @ K.T)
    visible = np.arange(L)[None, :] <= (first_pos + np.arange(n))[:, None]
    scores = np.where(visible, scores, -np.inf)
    w = np.exp(scores - scores.max(axis=1, keepdims=True))   # exp(-inf) = 0
    return (w @ V) / w.sum(axis=1, keepdims=True)


def prefill(query, k_pool, v_pool, block_tables, context_lens, query_start, scale) -> np.ndarray:
    """Paged attention of a chunk of new tokens per sequence (fp64, [T, Hq, D]).

    Sequence s owns query rows query_start[s] .. query_start[s+1]-1: its
    n = query_start[s+1] - query_start[s] newest tokens, at positions L-n ..
    L-1 where L = context_lens[s] counts every cached token including these
    (their keys and values are already in the pool). New token j attends over
    positions 0 .. L-n+j: every earlier token of the sequence, cached prefix
    included, and itself ([L], "How PagedAttention works", step 1: the prompt
    is stored in the request's blocks; step 4: attention walks the table).
    Written per (sequence, query head) as one masked attention of all n rows.
    """
    T, Hq, D = query.shape
    NB, Hkv, B, Dk = k_pool.shape
    if Dk != D or Hq % Hkv:
        raise ValueError("shape mismatch")
    G = Hq // Hkv
    qs = np.asarray(query_start, dtype=np.int64)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in range(len(context_lens)):
        L = int(context_lens[s])
        n = int(qs[s + 1] - qs[s])
        if n < 0 or n > L or L > block_tables.shape[1] * B:
            raise ValueError("bad query range or context length")
        if n == 0:
            continue
        Kc = gather(k_pool, block_tables[s], L, B).astype(np.float64)
        Vc = gather(v_pool, block_tables[s], L, B).astype(np.float64)
        rows = slice(int(qs[s]), int(qs[s]) + n)
        for h in range(Hq):
            g = h // G
            out[rows, h] = causal_attention(query[rows, h], Kc[g], Vc[g], L - n, scale)
    return out
