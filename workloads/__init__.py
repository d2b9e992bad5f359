"""Seeded synthetic inputs for paged KV-cache decode.

Both sides of every parity check draw their inputs from this module: the HIP
library's tests and benchmark, and the CPU oracle. It therefore holds none of
the method's arithmetic: no attention, no cache writes or block copies, no
token-to-slot translation. It draws context lengths, shuffled physical block
ids and fp16 N(0, 1) tensors, and lays the drawn ids out as block-table rows.

The one piece of block geometry it uses is part of the input recipe: a row
that must hold L tokens receives ceil(L / B) ids, and a pool is sized as a
multiple of the blocks all rows need. Everything that depends on where a token
lands inside those blocks is left to the code under test and to the oracle.

Conventions shared by all generators:
  * rng = numpy.random.default_rng(seed); fp16 values are float32 standard
    normals rounded to fp16 (round to nearest even).
  * physical ids come from one rng.permutation(NB), consumed in sequence order;
    unused table entries are -1.
  * pools are [NB, Hkv, B, D] fp16 and every slot, used or not, is drawn.
  * query is [S, Hq, D]; the new token's key/value are [S, Hkv, D] and belong
    at position L - 1 of each sequence (the context length counts the token
    being decoded).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

HEAD_DIM = 128


def f16_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """fp32 standard normals rounded to fp16."""
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def row_len(L: int, B: int) -> int:
    """Ids a table row receives for L tokens (input recipe: ceil(L / B))."""
    return -(-int(L) // int(B))


def pool_blocks(needed: int, num: int = 5, den: int = 4) -> int:
    """ceil(needed * num / den) in integers; default 1.25x headroom."""
    return -(-needed * num // den)


def lay_out_tables(lengths, B: int, ids: np.ndarray, MB: Optional[int] = None):
    """Give each sequence the next row_len(L, B) ids from `ids`, in order.

    Returns (tables int32 [S, MB] padded with -1, number of ids consumed).
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    rows = [row_len(L, B) for L in lengths]
    if MB is None:
        MB = max(rows) if rows else 1
    MB = max(int(MB), 1)
    tables = np.full((len(lengths), MB), -1, dtype=np.int32)
    off = 0
    for s, n in enumerate(rows):
        if n > MB:
            raise ValueError(f"sequence {s} needs {n} blocks > MB={MB}")
        tables[s, :n] = ids[off:off + n]
        off += n
    if off > len(ids):
        raise ValueError("not enough block ids")
    return tables, off


@dataclass
class DecodeCase:
    """One decode step's inputs for one layer."""
    name: str
    seed: int
    S: int
    Hq: int
    Hkv: int
    D: int
    B: int
    NB: int
    context_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray          # int32 [S, MB]
    query: np.ndarray                 # fp16 [S, Hq, D]
    key_new: np.ndarray               # fp16 [S, Hkv, D]  (token at L-1)
    value_new: np.ndarray             # fp16 [S, Hkv, D]
    k_pool: Optional[np.ndarray] = None   # fp16 [NB, Hkv, B, D]
    v_pool: Optional[np.ndarray] = None
    scale: float = 1.0 / np.sqrt(HEAD_DIM)
    extra: dict = field(default_factory=dict)

    @property
    def MB(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.S else 0

    def kv_bytes(self) -> int:
        """Counted KV bytes one decode reads: valid tokens x Hkv x D x (K and V) x 2 B."""
        return int(self.context_lens.astype(np.int64).sum()) * self.Hkv * self.D * 2 * 2


def make_case(name, seed, lengths, Hq, Hkv, B, D=HEAD_DIM, NB=None, pool_factor=(5, 4),
              MB=None, with_pools=True) -> DecodeCase:
    """Generic case: draw order is permutation, pools (K then V), query, new K, new V."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int32)
    return _finish_case(name, seed, rng, lengths, Hq, Hkv, B, D, NB, pool_factor, MB, with_pools)


def _finish_case(name, seed, rng, lengths, Hq, Hkv, B, D, NB, pool_factor, MB, with_pools):
    S = len(lengths)
    needed = sum(row_len(L, B) for L in lengths)
    if NB is None:
        NB = max(pool_blocks(needed, *pool_factor), 1)
    perm = rng.permutation(NB).astype(np.int32)
    tables, _ = lay_out_tables(lengths, B, perm, MB)
    k_pool = v_pool = None
    if with_pools:
        k_pool = f16_normal(rng, (NB, Hkv, B, D))
        v_pool = f16_normal(rng, (NB, Hkv, B, D))
    query = f16_normal(rng, (S, Hq, D))
    key_new = f16_normal(rng, (S, Hkv, D))
    value_new = f16_normal(rng, (S, Hkv, D))
    return DecodeCase(name=name, seed=seed, S=S, Hq=Hq, Hkv=Hkv, D=D, B=B, NB=int(NB),
                      context_lens=lengths, block_tables=tables, query=query,
                      key_new=key_new, value_new=value_new, k_pool=k_pool, v_pool=v_pool)


# ---------------------------------------------------------------------------
# The five workloads. Shapes follow the pages' examples: a 7B/8B-class layer
# (32 KV heads of 128 dims, fp16), blocks of 16 tokens, request lengths drawn
# uniformly as in the lesson's simulation and the blog's chat example.
# ---------------------------------------------------------------------------

def tiny_worked_example(seed: int = 1) -> DecodeCase:
    """Two sequences of 40 and 48 tokens, 4 heads, a 16-block pool, B = 16.

    Seq 0 gets the first three ids of permutation(16), seq 1 the next three.
    """
    rng = np.random.default_rng(seed)
    lengths = np.array([40, 48], dtype=np.int32)
    return _finish_case("tiny_worked_example", seed, rng, lengths, 4, 4, 16, HEAD_DIM,
                        16, (5, 4), None, True)


def growth_example(seed: int = 11) -> dict:
    """The lesson's life-of-a-request walk: a 40-token prompt in physical blocks
    7, 2, 9 of a 16-block pool; nine more tokens (positions 40..48) arrive, the
    last of which needs the freshly allocated block 4.

    Returns pools, the 3- and 4-entry tables, the nine new tokens' K/V and a query.
    """
    rng = np.random.default_rng(seed)
    Hq = Hkv = 4
    B, NB, D = 16, 16, HEAD_DIM
    k_pool = f16_normal(rng, (NB, Hkv, B, D))
    v_pool = f16_normal(rng, (NB, Hkv, B, D))
    new_k = f16_normal(rng, (9, Hkv, D))
    new_v = f16_normal(rng, (9, Hkv, D))
    query = f16_normal(rng, (1, Hq, D))
    return dict(Hq=Hq, Hkv=Hkv, B=B, NB=NB, D=D, k_pool=k_pool, v_pool=v_pool,
                table_before=np.array([[7, 2, 9]], dtype=np.int32),
                table_after=np.array([[7, 2, 9, 4]], dtype=np.int32),
                len_before=40, len_after=49,
                positions=np.arange(40, 49, dtype=np.int32),
                new_k=new_k, new_v=new_v, query=query, scale=1.0 / np.sqrt(D))


def seven_b_single_layer(seed: int = 7) -> DecodeCase:
    """Batch 8, lengths uniform in [50, 900) (the lesson's seed-7 draw),
    32 heads, B = 16, pool = 1.25x the blocks needed."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(50, 900, size=8).astype(np.int32)
    return _finish_case("7b_single_layer", seed, rng, lengths, 32, 32, 16, HEAD_DIM,
                        None, (5, 4), None, True)


CHAT_SEED = 3
CHAT_LAYERS = 32


def chat_lengths(seed: int = CHAT_SEED, S: int = 128) -> np.ndarray:
    """Prompt uniform in [100, 2000] plus generation uniform in [50, 500]."""
    rng = np.random.default_rng(seed)
    prompt = rng.integers(100, 2001, size=S)
    gen = rng.integers(50, 501, size=S)
    return (prompt + gen).astype(np.int32)


def chat_layer(layer: int, seed: int = CHAT_SEED, S: int = 128, with_pools: bool = False,
               lengths: Optional[np.ndarray] = None, B: int = 16,
               contiguous: bool = False, Hq: int = 32, Hkv: int = 32) -> DecodeCase:
    """One layer of the batch-128 chat workload (32 heads, B = 16, 1.25x pool).

    All layers share the lengths; each layer has its own shuffle, query and new
    K/V (rng seeded with seed * 1000 + layer). `B` changes the block size;
    `contiguous=True` gives every sequence one block as long as the longest
    sequence (the pre-paging layout), in a pool of exactly S blocks. `Hq` / `Hkv` change the
    head counts (grouped-query variants: 32 query heads over 8 KV heads, or 64 over 8). Pools are
    large (about 1.7 GB
    each), so by default they are not drawn here: `device_pools` draws them on
    the GPU. `with_pools=True` draws them on the host (slow; small S only).
    """
    if lengths is None:
        lengths = chat_lengths(seed, S)
    lengths = np.asarray(lengths, np.int32)
    rng = np.random.default_rng(seed * 1000 + layer)
    NB = None
    if contiguous:
        # the layout before paging: one region per sequence, sized for the
        # longest sequence of the batch (a multiple of 16 tokens)
        B = -(-int(lengths.max()) // 16) * 16
        NB = len(lengths)
    name = f"chat_b{S}_layer{layer}" + ("" if (Hq, Hkv) == (32, 32) else f"_h{Hq}x{Hkv}")
    case = _finish_case(name, seed, rng, lengths, Hq, Hkv, B, HEAD_DIM, NB, (5, 4), None,
                        with_pools)
    case.extra["layer"] = layer
    return case


def chat_pool_seed(layer: int, seed: int = CHAT_SEED) -> int:
    """Seed of the device-drawn pools of one chat layer."""
    return seed * 1000 + layer


def device_pools(NB: int, Hkv: int, B: int, D: int, seed: int, device="cuda"):
    """K and V pools drawn on the device: torch N(0, 1) in fp32 rounded to fp16.

    Reproducible for a fixed torch/ROCm build; tests copy them back to the host
    for the oracle, so the exact draw never matters for parity.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    shape = (NB, Hkv, B, D)
    k = torch.empty(shape, dtype=torch.float16, device=device)
    v = torch.empty(shape, dtype=torch.float16, device=device)
    # draw in chunks of blocks to bound the fp32 temporary
    step = max(1, (1 << 26) // (Hkv * B * D))
    for pool in (k, v):
        for b0 in range(0, NB, step):
            b1 = min(NB, b0 + step)
            pool[b0:b1] = torch.randn((b1 - b0,) + shape[1:], generator=g, device=device,
                                      dtype=torch.float32).to(torch.float16)
    return k, v


def shared_prefix(seed: int = 4, n_seq: int = 64, prefix_len: int = 500, Hq: int = 32,
                  Hkv: int = 8, B: int = 16, D: int = HEAD_DIM) -> dict:
    """64 samples of one 500-token prompt, each with a private suffix uniform in
    [50, 500]; grouped-query heads (32 query, 8 KV).

    The prompt fills ceil(500 / 16) = 32 shared blocks, the last one partly.
    Each sequence's first suffix token lands in that partly filled block, so
    every sequence first takes a private copy of it (the prompt's owner keeps
    its reference, so the count is never 1 when a sample writes). Returned:
      shared_ids   [32]  physical ids of the prompt's blocks
      private_ids  list of per-sequence id arrays: the copy target first, then
                   the blocks its suffix needs beyond block 31
      copy_pairs   int32 [64, 2] (src = shared block 31, dst = private copy)
      tables       int32 [64, MB] after the copy (31 shared ids, then private)
      context_lens int32 [64] = 500 + suffix
      suffix_k/v   per sequence fp16 [L - 500, Hkv, D], positions 500 .. L-1;
                   the last row is the token decoded in the step
    """
    rng = np.random.default_rng(seed)
    suffix = rng.integers(50, 501, size=n_seq)
    lengths = (prefix_len + suffix).astype(np.int32)
    n_prefix = row_len(prefix_len, B)
    partial = prefix_len % B != 0
    n_shared_kept = n_prefix - 1 if partial else n_prefix
    private_counts = [row_len(L, B) - n_shared_kept for L in lengths]
    needed = n_prefix + sum(private_counts)
    NB = pool_blocks(needed)
    perm = rng.permutation(NB).astype(np.int32)
    shared_ids = perm[:n_prefix]
    off = n_prefix
    private_ids = []
    for c in private_counts:
        private_ids.append(perm[off:off + c])
        off += c
    MB = max(row_len(L, B) for L in lengths)
    tables = np.full((n_seq, MB), -1, dtype=np.int32)
    for s in range(n_seq):
        row = np.concatenate([shared_ids[:n_shared_kept], private_ids[s]])
        tables[s, :len(row)] = row
    copy_pairs = np.zeros((n_seq if partial else 0, 2), dtype=np.int32)
    if partial:
        copy_pairs[:, 0] = shared_ids[-1]
        copy_pairs[:, 1] = [p[0] for p in private_ids]
    k_pool = f16_normal(rng, (NB, Hkv, B, D))
    v_pool = f16_normal(rng, (NB, Hkv, B, D))
    query = f16_normal(rng, (n_seq, Hq, D))
    suffix_k = [f16_normal(rng, (int(n), Hkv, D)) for n in suffix]
    suffix_v = [f16_normal(rng, (int(n), Hkv, D)) for n in suffix]
    return dict(S=n_seq, Hq=Hq, Hkv=Hkv, B=B, D=D, NB=NB, prefix_len=prefix_len,
                shared_ids=shared_ids, private_ids=private_ids, copy_pairs=copy_pairs,
                tables=tables, context_lens=lengths, k_pool=k_pool, v_pool=v_pool,
                query=query, suffix_k=suffix_k, suffix_v=suffix_v, scale=1.0 / np.sqrt(D))


def long_context(seed: int = 5, with_pools: bool = True) -> DecodeCase:
    """Batch 16 at 4096 tokens, 32 heads, B = 32, pool of exactly 2048 blocks,
    fully shuffled. The host pools take about 30 s to draw; with
    `with_pools=False` they are left to `device_pools` (seed * 1000)."""
    rng = np.random.default_rng(seed)
    lengths = np.full(16, 4096, dtype=np.int32)
    return _finish_case("long_context_b16_4096", seed, rng, lengths, 32, 32, 32, HEAD_DIM,
                        2048, (5, 4), None, with_pools)


# ---------------------------------------------------------------------------
# Prefill inputs: a chunk of new tokens per sequence. Sequence s holds
# cached_lens[s] + new_lens[s] tokens in the pools (every slot drawn), its new
# tokens are the last new_lens[s]; their queries are packed row after row.
# ---------------------------------------------------------------------------

@dataclass
class PrefillCase:
    name: str
    seed: int
    S: int
    Hq: int
    Hkv: int
    D: int
    B: int
    NB: int
    context_lens: np.ndarray          # int32 [S]   cached + new
    new_lens: np.ndarray              # int32 [S]
    query_start: np.ndarray           # int32 [S + 1]
    block_tables: np.ndarray          # int32 [S, MB]
    query: np.ndarray                 # fp16 [T, Hq, D]
    k_pool: Optional[np.ndarray] = None
    v_pool: Optional[np.ndarray] = None
    scale: float = 1.0 / np.sqrt(HEAD_DIM)

    @property
    def T(self) -> int:
        return int(self.query_start[-1])

    @property
    def MB(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_query_len(self) -> int:
        return int(self.new_lens.max()) if self.S else 0


def make_prefill_case(name, seed, new_lens, cached_lens, Hq, Hkv, B, D=HEAD_DIM, NB=None,
                      with_pools=True) -> PrefillCase:
    """Draw order: permutation, pools (K then V), packed query."""
    rng = np.random.default_rng(seed)
    new_lens = np.asarray(new_lens, dtype=np.int32)
    lengths = (np.asarray(cached_lens, dtype=np.int32) + new_lens).astype(np.int32)
    S = len(lengths)
    needed = sum(row_len(L, B) for L in lengths)
    if NB is None:
        NB = max(pool_blocks(needed), 1)
    perm = rng.permutation(NB).astype(np.int32)
    tables, _ = lay_out_tables(lengths, B, perm)
    k_pool = v_pool = None
    if with_pools:
        k_pool = f16_normal(rng, (NB, Hkv, B, D))
        v_pool = f16_normal(rng, (NB, Hkv, B, D))
    qs = np.zeros(S + 1, dtype=np.int32)
    qs[1:] = np.cumsum(new_lens)
    query = f16_normal(rng, (int(qs[-1]), Hq, D))
    return PrefillCase(name=name, seed=seed, S=S, Hq=Hq, Hkv=Hkv, D=D, B=B, NB=int(NB),
                       context_lens=lengths, new_lens=new_lens, query_start=qs,
                       block_tables=tables, query=query, k_pool=k_pool, v_pool=v_pool,
                       scale=1.0 / np.sqrt(D))


CHAT_PREFILL_SEED = 6


def chat_prefill(seed: int = CHAT_PREFILL_SEED, S: int = 16, with_pools: bool = True) -> PrefillCase:
    """Prompt processing for the chat endpoint: S prompts with lengths uniform in
    [100, 2000] (the blog's chat example), nothing cached, 32 query heads = 32
    KV heads of 128 dims, B = 16, pool 1.25x the blocks needed."""
    rng = np.random.default_rng(seed)
    prompts = rng.integers(100, 2001, size=S).astype(np.int32)
    return make_prefill_case(f"chat_prefill_s{S}", seed * 1000 + 1, prompts, np.zeros(S, np.int32),
                             32, 32, 16, with_pools=with_pools)


def prefix_prefill(seed: int = 4, n_seq: int = 64) -> dict:
    """The shared-prefix workload (shared_prefix: a cached 500-token prompt,
    grouped heads 32/8) processed as prefill: each sequence's private suffix is
    the chunk of new tokens. Adds the packed suffix queries (fp16 [T, Hq, D],
    drawn from default_rng(seed * 1000 + 1)) and query_start [S + 1] to the
    shared_prefix dict."""
    w = shared_prefix(seed=seed, n_seq=n_seq)
    n = (w["context_lens"] - w["prefix_len"]).astype(np.int32)
    qs = np.zeros(len(n) + 1, dtype=np.int32)
    qs[1:] = np.cumsum(n)
    rng = np.random.default_rng(seed * 1000 + 1)
    w["prefill_query"] = f16_normal(rng, (int(qs[-1]), w["Hq"], w["D"]))
    w["query_start"] = qs
    w["new_lens"] = n
    return w
