"""Peaked score distributions for the GPU parity tests (test infrastructure).

The seeded workloads draw queries and keys as N(0, 1) at scale 1/sqrt(128), so
every score sits within a few units of the others and the softmax is nearly
flat. Real attention is peaked: a few tokens (recent ones, sink tokens, a
token that repeats the query's content) score far above the rest. The pages
state that paging changes no output ([L] "Paged Attention: OS-Inspired Memory
Management for KV Caches", "How PagedAttention works", step 4, and "Key
takeaways": paging is exact), so peaked inputs must match the oracle as well.
These helpers turn a seeded case into such inputs:

  dominant keys  a few late keys are set to a multiple of a direction the
                 queries share, so that each scores far above every earlier key
                 (the closed form: with one such key the output is that
                 token's value row);
  ramp           every key gets a component along that direction that grows
                 with its position, so scores rise steadily along the walk;
  scale          the caller's scale, e.g. 1.0 or negative, on N(0, 1) inputs.

Keys are placed at their logical positions through the case's block table with
the oracle's slot geometry; the new decode token (position L - 1) is edited in
the case's key_new, since pa_write_kv stores it during the step. The helpers
also report, from the fp64 scores, how often a running maximum walked in
16-token units must rise by more than 2^8 after a wave's first unit, which is
when the matrix-core kernels' lazy rescaling runs.
"""
from __future__ import annotations

import numpy as np

import oracle

LOG2E = 1.4426950408889634
UNIT = 16          # tokens per kernel work unit
SLACK = 8.0        # log2 units a running maximum may fall behind before it is raised


def _set_key(pool, table_row, t, B, g, vec):
    slot = oracle.slot_of(table_row, t, B)
    pool[slot // B, g, slot % B, :] = vec


def _key(pool, table_row, t, B, g):
    slot = oracle.slot_of(table_row, t, B)
    return pool[slot // B, g, slot % B, :]


def _f16(x):
    return np.asarray(x, np.float64).astype(np.float16)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def _decode_direction(case, s, g):
    """The mean query of KV head g's group: every head of the group has a
    positive dot product with it."""
    G = case.Hq // case.Hkv
    return case.query[s, g * G:(g + 1) * G].astype(np.float64).mean(axis=0)


def _decode_edit(case, s, t, g, fn):
    """Replace key (s, t, g) by fn(old key as fp64)."""
    L = int(case.context_lens[s])
    if t == L - 1:
        case.key_new[s, g] = _f16(fn(case.key_new[s, g].astype(np.float64)))
    else:
        old = _key(case.k_pool, case.block_tables[s], t, case.B, g).astype(np.float64)
        _set_key(case.k_pool, case.block_tables[s], t, case.B, g, _f16(fn(old)))


def decode_dominant_keys(case, rng, n_keys=3, first_gap=12.0, step=6.0):
    """n_keys late keys per (sequence, KV head), at increasing positions, each
    scoring about `step` log2 units above the previous one and the first about
    `first_gap` above the typical score: every one of them raises the running
    maximum of the wave that reads it. Returns the positions per (s, g)."""
    where = {}
    for s in range(case.S):
        L = int(case.context_lens[s])
        if L < 2:
            continue
        lo = max(1, (2 * L) // 5)
        k = min(n_keys, L - lo)
        pos = np.sort(rng.choice(np.arange(lo, L), size=k, replace=False))
        for g in range(case.Hkv):
            d = _decode_direction(case, s, g)
            dd = float(d @ d)
            for i, t in enumerate(pos.tolist()):
                # score of the mean query: scale * c * |d|^2 = target (natural units)
                target = (first_gap + i * step) / LOG2E
                c = target / (case.scale * dd)
                _decode_edit(case, s, t, g, lambda old, c=c, d=d: c * d)
            where[(s, g)] = pos
    return where


def decode_ramp(case, rise_log2=18.0):
    """Adds to key t of every (sequence, KV head) a component along the group's
    mean query that grows linearly with t, so that the mean query's score
    rises by about rise_log2 log2 units from the first to the last token."""
    for s in range(case.S):
        L = int(case.context_lens[s])
        if L < 2:
            continue
        for g in range(case.Hkv):
            d = _decode_direction(case, s, g)
            c = rise_log2 / LOG2E / (case.scale * float(d @ d))
            for t in range(L):
                f = c * t / (L - 1)
                _decode_edit(case, s, t, g, lambda old, f=f, d=d: old + f * d)


def decode_scores_log2(case, s, h):
    """fp64 scores of query head h of sequence s over its L tokens, in log2
    units, after the step's write of the new token."""
    G = case.Hq // case.Hkv
    g = h // G
    L = int(case.context_lens[s])
    K = oracle.gather(case.k_pool, case.block_tables[s], L, case.B)[g].astype(np.float64)
    K[L - 1] = case.key_new[s, g].astype(np.float64)
    return case.scale * LOG2E * (K @ case.query[s, h].astype(np.float64))


def lazy_rescale_walks(scores, P, waves=4):
    """Among the walks a decode partition kernel makes over one (sequence,
    head) -- each partition of P tokens, its 16-token units dealt round-robin
    to `waves` waves -- count those whose running maximum must be raised
    after the wave's first unit (a later unit's maximum above it by more than
    SLACK). Returns (walks with such a rise, walks with more than one unit)."""
    L = len(scores)
    rises = multi = 0
    for p0 in range(0, L, P):
        part = scores[p0:min(L, p0 + P)]
        units = [part[u:u + UNIT].max() for u in range(0, len(part), UNIT)]
        for w in range(waves):
            mine = units[w::waves]
            if len(mine) < 2:
                continue
            multi += 1
            m = mine[0]
            hit = False
            for x in mine[1:]:
                if x > m + SLACK:
                    hit = True
                    m = x
            rises += hit
    return rises, multi


def decode_rescale_count(case, P, waves=4):
    """lazy_rescale_walks summed over every (sequence, query head)."""
    rises = multi = 0
    for s in range(case.S):
        if int(case.context_lens[s]) == 0:
            continue
        for h in range(case.Hq):
            r, m = lazy_rescale_walks(decode_scores_log2(case, s, h), P, waves)
            rises += r
            multi += m
    return rises, multi


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def prefill_shared_direction(case, rng, weight=1.0):
    """Adds weight * u_{s,g} (one fp16 N(0, 1) vector per sequence and KV head)
    to every query row of that sequence and group, so that a key along u scores
    high for all of them. Returns {(s, g): u}."""
    G = case.Hq // case.Hkv
    qs = case.query_start
    dirs = {}
    for s in range(case.S):
        r0, r1 = int(qs[s]), int(qs[s + 1])
        for g in range(case.Hkv):
            u = rng.standard_normal(case.D).astype(np.float16).astype(np.float64)
            dirs[(s, g)] = u
            q = case.query[r0:r1, g * G:(g + 1) * G].astype(np.float64) + weight * u
            case.query[r0:r1, g * G:(g + 1) * G] = _f16(q)
    return dirs


def prefill_dominant_keys(case, rng, dirs, n_keys=3, first_gap=14.0, step=8.0):
    """n_keys keys per (sequence, KV head) at increasing positions spread over
    the sequence, each along u with a score about first_gap + i * step log2
    units for a query near u."""
    for s in range(case.S):
        L = int(case.context_lens[s])
        if L < 2:
            continue
        k = min(n_keys, L - 1)
        pos = np.sort(rng.choice(np.arange(1, L), size=k, replace=False))
        for g in range(case.Hkv):
            u = dirs[(s, g)]
            for i, t in enumerate(pos.tolist()):
                c = (first_gap + i * step) / LOG2E / (abs(case.scale) * float(u @ u))
                vec = np.sign(case.scale) * c * u
                _set_key(case.k_pool, case.block_tables[s], t, case.B, g, _f16(vec))


def prefill_ramp(case, dirs, rise_log2=18.0):
    """Key t of every (sequence, KV head) gains a component along u growing
    linearly with t: scores of queries near u rise by about rise_log2 log2
    units over the sequence."""
    for s in range(case.S):
        L = int(case.context_lens[s])
        if L < 2:
            continue
        for g in range(case.Hkv):
            u = dirs[(s, g)]
            c = rise_log2 / LOG2E / (case.scale * float(u @ u))
            for t in range(L):
                old = _key(case.k_pool, case.block_tables[s], t, case.B, g).astype(np.float64)
                _set_key(case.k_pool, case.block_tables[s], t, case.B, g,
                         _f16(old + c * t / (L - 1) * u))


def prefill_rescale_rows(case, chunk=32):
    """Rows (and heads) whose maximum score over the keys they see exceeds the
    maximum over the first `chunk` keys by more than SLACK log2 units: rows
    for which a running maximum walked chunk by chunk must be raised after its
    first chunk. Returns (such (row, head) pairs, all (row, head) pairs)."""
    G = case.Hq // case.Hkv
    qs = case.query_start
    hits = total = 0
    for s in range(case.S):
        L = int(case.context_lens[s])
        r0, r1 = int(qs[s]), int(qs[s + 1])
        n = r1 - r0
        if n == 0:
            continue
        K = oracle.gather(case.k_pool, case.block_tables[s], L, case.B).astype(np.float64)
        for h in range(case.Hq):
            sc = case.scale * LOG2E * (case.query[r0:r1, h].astype(np.float64) @ K[h // G].T)
            for j in range(n):
                p = L - n + j
                first = sc[j, :min(chunk, p + 1)].max()
                hits += bool(sc[j, :p + 1].max() > first + SLACK)
                total += 1
    return hits, total
