"""Benchmark: paged decode on one MI355X.

Default workload (`--workload chat`): 128 sequences, context = prompt
U[100, 2000] + generated U[50, 500] tokens, 32 layers, each with its own K/V
block pool (32 KV heads, head dim 128, fp16, blocks of 16 tokens, 1.25x pool,
shuffled physical ids). One step is one decode step of the whole model's
attention cache path: per layer, the new token's slot and K/V store
(pa_append_kv, the slot mapping and store in one launch) and paged decode
attention (pa_decode).

Other workloads (`--workload 7b|shared_prefix|long_context|tiny`) time one
layer per step and rotate over `--replicas` copies of the inputs so that the
small ones are read from HBM rather than from the caches (`--replicas 1`
measures them cache-warm). The shared-prefix workload also times its
copy-on-write `pa_copy_blocks` (64 pairs) separately.

Inputs are synthetic (seeded) and resident in HBM before the timed region.
Prints one JSON line. `value` is KV bytes read per step (valid tokens x KV
heads x 128 x K and V x 2 B, summed over the step's layers) divided by the step
time. `roofline` prices one pa_decode call (partition + reduce kernels), timed
with HIP events on the stream it runs on, against 8 TB/s. `cpu_baseline` times
the CPU oracle on a bounded sample of the same workload.

Prefill (`--workload prefill`: 16 chat prompts, nothing cached; `--workload
prefix_prefill`: 64 suffixes after a shared cached prompt, grouped heads) times
the prompt tokens' K/V stores and pa_prefill per step and prices the pa_prefill
launch against the fp16 matrix-core peak. `--workload swap` and
`--workload block_manager` time pa_swap_blocks and the host block manager.
`--graph` replays each decode step as a HIP graph.

    python bench.py [--workload chat] [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged-decode KV-read GB/s (% of HBM peak) + decode tokens/s, batch 128"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 10; prefill 50: one step is under a millisecond)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default 3; prefill 50, so that the clock has "
                         "ramped up before the timed region)")
    ap.add_argument("--workload", default="chat",
                    choices=["chat", "7b", "shared_prefix", "long_context", "tiny", "block_manager",
                             "swap", "prefill", "prefix_prefill"])
    ap.add_argument("--layers", type=int, default=32, help="chat workload: layers per step")
    ap.add_argument("--block-size", type=int, default=16, help="chat workload: tokens per block")
    ap.add_argument("--q-heads", type=int, default=32, help="chat workload: query heads")
    ap.add_argument("--kv-heads", type=int, default=32,
                    help="chat workload: KV heads (8 with 32 or 64 query heads: grouped-query "
                         "variants)")
    ap.add_argument("--contiguous", action="store_true",
                    help="chat workload: one block per sequence sized for the longest one "
                         "(the pre-paging layout), for comparison")
    ap.add_argument("--replicas", type=int, default=0,
                    help="other workloads: input copies rotated over steps (0 = enough to "
                         "exceed the 256 MB last-level cache; 1 = cache-warm)")
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--graph", action="store_true",
                    help="decode workloads: capture each input set's step (all layers: slot "
                         "mapping, K/V store, decode) in a HIP graph and time graph replays; the "
                         "per-call roofline events stay eager")
    ap.add_argument("--prompts", type=int, default=16, help="prefill workload: prompts per step")
    ap.add_argument("--cpu-sample-layers", type=int, default=4,
                    help="chat workload: layers the oracle decodes for cpu_baseline, evenly spaced "
                         "(32 = every layer of the step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-reference-mb", type=int, default=0,
                    help="after timing, run one plain device-to-device copy of this many MiB "
                         "(a copy of known size for scaling traffic counters)")
    args = ap.parse_args()
    short = args.workload in ("prefill", "prefix_prefill")
    if args.steps is None:
        args.steps = 50 if short else 10
    if args.warmup is None:
        args.warmup = 50 if short else 3
    return args


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pa_decode_chat_b128_traffic.json")


def _sources_hash(rel_paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in rel_paths:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode launch from the committed counter summary, or None
    when a source it lists (the decode kernels, their header, the build
    flags) changed after the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("decode_source_sha256") != _sources_hash(t["sources"]):
            return None
    except (OSError, ValueError, KeyError):
        return None
    return t.get("traffic_bytes_per_launch")


PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pa_prefill_chat_s16_traffic.json")


def prefill_measured_traffic():
    """HBM bytes per prefill launch from the committed counter summary, or None
    when the prefill kernel or its build flags changed after the counters were taken."""
    try:
        with open(PREFILL_TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("prefill_source_sha256") != _sources_hash(t["sources"]):
            return None
    except (OSError, ValueError, KeyError):
        return None
    return t.get("traffic_bytes_per_launch")


def copy_reference(mb):
    """One plain device-to-device copy of exactly mb MiB (torch copy_, a memory
    copy), after the timed region: the known-size reference that scales the
    FETCH_SIZE and WRITE_SIZE counters."""
    import torch
    a = torch.zeros(mb << 19, dtype=torch.float16, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy reference: {mb << 20} B read, {mb << 20} B written")


# ---------------------------------------------------------------------------
# workload set-up: a list of "layers", each one decode call's inputs on the GPU
# ---------------------------------------------------------------------------

def _upload(case, kp, vp, dev):
    import torch
    return dict(case=case, kp=kp, vp=vp, tables=dev(case.block_tables), lens=dev(case.context_lens),
                q=dev(case.query), k_new=dev(case.key_new), v_new=dev(case.value_new),
                slots=torch.empty(case.S, dtype=torch.int64, device="cuda"))


def _replicate(layer, n):
    out = [layer]
    for _ in range(n - 1):
        out.append({k: (v.clone() if hasattr(v, "clone") else v) for k, v in layer.items()})
    return out


def _replicas_for(args, bytes_per_layer):
    if args.replicas > 0:
        return args.replicas
    return max(1, int(np.ceil(1.0e9 / max(bytes_per_layer, 1))))   # > 1 GB in rotation


def build_chat(args, dev):
    import workloads as W
    lengths = W.chat_lengths()
    layers = []
    for layer in range(args.layers):
        c = W.chat_layer(layer, lengths=lengths, B=args.block_size, contiguous=args.contiguous,
                         Hq=args.q_heads, Hkv=args.kv_heads)
        kp, vp = W.device_pools(c.NB, c.Hkv, c.B, c.D, seed=W.chat_pool_seed(layer))
        layers.append(_upload(c, kp, vp, dev))
    desc = "chat decode, batch 128, 32 layers (prompt U[100,2000] + generated U[50,500])"
    if (args.q_heads, args.kv_heads) != (32, 32):
        desc += f" -- GROUPED heads: {args.q_heads} query / {args.kv_heads} KV"
    if args.layers != 32:
        desc += f" -- REDUCED to {args.layers} layers"
    if args.contiguous:
        desc += f" -- CONTIGUOUS layout (one {layers[0]['case'].B}-token block per sequence)"
    elif args.block_size != 16:
        desc += f" -- block size {args.block_size}"
    return [layers], desc, {}


def build_single(args, dev, case, desc):
    kp, vp = dev(case.k_pool), dev(case.v_pool)
    base = _upload(case, kp, vp, dev)
    pool_bytes = 2 * kp.numel() * 2
    reps = _replicas_for(args, pool_bytes)
    return [[x] for x in _replicate(base, reps)], desc, {"replicas": reps}


def build_shared_prefix(args, dev, pa):
    """Set-up runs the workload's own boundary calls: copy-on-write of the
    shared partial block for all 64 samples, then the suffix tokens up to
    position L-2. The timed step writes the last token and decodes."""
    import torch
    import workloads as W
    d = W.shared_prefix()
    case = W.DecodeCase(name="shared_prefix", seed=4, S=d["S"], Hq=d["Hq"], Hkv=d["Hkv"], D=d["D"],
                        B=d["B"], NB=d["NB"], context_lens=d["context_lens"], block_tables=d["tables"],
                        query=d["query"], key_new=np.stack([k[-1] for k in d["suffix_k"]]),
                        value_new=np.stack([v[-1] for v in d["suffix_v"]]), scale=d["scale"])
    kp, vp = dev(d["k_pool"]), dev(d["v_pool"])
    pairs = dev(d["copy_pairs"])
    pristine = (kp.clone(), vp.clone())
    pa.pa_copy_blocks(kp, vp, pairs)
    seq, pos, ks, vs = [], [], [], []
    for s in range(d["S"]):
        n = int(d["context_lens"][s]) - d["prefix_len"] - 1
        seq += [s] * n
        pos += list(range(d["prefix_len"], d["prefix_len"] + n))
        ks.append(d["suffix_k"][s][:-1])
        vs.append(d["suffix_v"][s][:-1])
    tables = dev(d["tables"])
    slots = pa.pa_slot_mapping(tables, d["B"], d["NB"], seq_ids=dev(np.array(seq, np.int32)),
                               positions=dev(np.array(pos, np.int32)))
    pa.pa_write_kv(dev(np.concatenate(ks)), dev(np.concatenate(vs)), kp, vp, slots)
    torch.cuda.synchronize()
    base = _upload(case, kp, vp, dev)
    reps = _replicas_for(args, 2 * kp.numel() * 2)
    extra = {"replicas": reps, "copy": (pristine, pairs, d)}
    desc = ("shared prefix: 64 samples of a 500-token prompt + suffix U[50,500], "
            "32 query / 8 KV heads, B=16")
    return [[x] for x in _replicate(base, reps)], desc, extra


def time_copy_on_write(pa, extra):
    """pa_copy_blocks of the 64 copy-on-write pairs, on a scratch copy."""
    import torch
    (k0, v0), pairs, d = extra["copy"]
    kp, vp = k0.clone(), v0.clone()
    for _ in range(3):
        pa.pa_copy_blocks(kp, vp, pairs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 20
    e0.record()
    for _ in range(n):
        pa.pa_copy_blocks(kp, vp, pairs)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    moved = 2 * 2 * pairs.shape[0] * d["Hkv"] * d["B"] * d["D"] * 2   # read + write, K and V
    return {"pairs": int(pairs.shape[0]), "us": round(us, 2),
            "bytes_read_plus_written": moved, "GBs": round(moved / us / 1e3, 1)}


def bench_block_manager(args):
    """Host block manager (pa_bm_*): the bookkeeping of one decode step of the
    batch-128 chat workload -- one token appended to each sequence, then the
    batch's block tables and lengths exported for pa_decode. The oracle's
    Python manager does the same steps as the CPU baseline."""
    import paged_kv_cache_151_amd as pa
    import oracle
    import workloads as W
    lengths = W.chat_lengths()
    S, B = len(lengths), 16
    NB = W.pool_blocks(sum(W.row_len(L, B) for L in lengths))
    MB = W.row_len(int(lengths.max()) + args.steps + args.warmup + 1, B)
    m = pa.BlockManager(NB, B)
    seqs = [m.add_sequence() for _ in range(S)]
    t0 = time.perf_counter()
    for sid, L in zip(seqs, lengths):
        m.append_tokens([sid] * (int(L) - 1))
    prefill_s = time.perf_counter() - t0
    ids = np.array(seqs, np.int32)
    for _ in range(args.warmup):
        m.append_tokens(ids)
        m.export(ids, MB)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        m.append_tokens(ids)
        m.export(ids, MB)
    us = (time.perf_counter() - t0) / args.steps * 1e6
    # the oracle's manager on the same work (prefill excluded from its timing too)
    ref = oracle.BlockManager(NB, B)
    seqs_ref = [ref.new_sequence() for _ in range(S)]
    for q, L in zip(seqs_ref, lengths):
        for _ in range(int(L) - 1):
            ref.append(q)
    n_ref = max(1, min(args.steps, 20))
    t0 = time.perf_counter()
    for _ in range(n_ref):
        for q in seqs_ref:
            ref.append(q)
        np.array([q.blocks + [-1] * (MB - len(q.blocks)) for q in seqs_ref], np.int32)
    ref_us = (time.perf_counter() - t0) / n_ref * 1e6
    res = {
        "metric": "host block manager: one decode step of bookkeeping (append + export), batch 128",
        "value": round(us, 2), "unit": "us/step", "n_gpus": 0, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": False, "data": "synthetic",
        "config": {"workload": "chat lengths (prompt U[100,2000] + generated U[50,500]), 128 sequences",
                   "pool_blocks": NB, "block_size": B, "table_width": MB,
                   "prefill_tokens": int((lengths - 1).sum()), "prefill_s": round(prefill_s, 3)},
        "cpu_baseline": {"value": round(ref_us, 1), "unit": "us/step", "cores": 1, "kind": "oracle",
                         "sample": f"oracle's Python manager, {n_ref} steps"},
    }
    print(json.dumps(res), flush=True)


def bench_swap(args):
    """pa_swap_blocks between the chat workload's device pool (layer 0) and a
    pinned host pool: 4096 blocks of 32 heads x 16 tokens x 128 dims fp16
    (128 KiB per pool each, 1 GiB of K + V per direction)."""
    import torch
    import paged_kv_cache_151_amd as pa
    import workloads as W
    torch.cuda.set_device(0)
    c = W.chat_layer(0)
    kp, vp = W.device_pools(c.NB, c.Hkv, c.B, c.D, seed=W.chat_pool_seed(0))
    n = 4096
    host_k = torch.empty((n, c.Hkv, c.B, c.D), dtype=torch.float16).pin_memory()
    host_v = torch.empty_like(host_k).pin_memory()
    rng = np.random.default_rng(0)
    dev_ids = rng.permutation(c.NB)[:n].astype(np.int32)
    out_pairs = torch.from_numpy(np.stack([dev_ids, np.arange(n, dtype=np.int32)], 1)).cuda()
    in_pairs = torch.from_numpy(np.stack([np.arange(n, dtype=np.int32),
                                          rng.permutation(c.NB)[:n].astype(np.int32)], 1)).cuda()
    block_bytes = c.Hkv * c.B * c.D * 2
    moved = 2 * n * block_bytes
    res = {}
    for name, fn in (("out", lambda: pa.pa_swap_blocks(host_k, host_v, kp, vp, out_pairs)),
                     ("in", lambda: pa.pa_swap_blocks(kp, vp, host_k, host_v, in_pairs))):
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        res[name] = {"ms": round(ms, 3), "GBs": round(moved / ms / 1e6, 1)}
    print(json.dumps({
        "metric": "pa_swap_blocks host-link GB/s (device pool <-> pinned host pool)",
        "value": res["out"]["GBs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "data": "synthetic",
        "config": {"workload": "4096 blocks of the chat workload's layer-0 pool (32 heads x 16 tokens x "
                               "128 dims fp16), K and V", "bytes_per_direction": moved},
        "swap_out": res["out"], "swap_in": res["in"]}), flush=True)


MFMA_F16_PEAK_TFLOPS = 2500.0


def prefill_flops(new_lens, context_lens, Hq, D):
    """Algorithmic flops of causal paged prefill: a new token at position p
    scores p + 1 keys and sums p + 1 values, 2 D flops each, per query head."""
    total = 0
    for n, L in zip(new_lens.tolist(), context_lens.tolist()):
        first = L - n + 1                      # keys seen by the first new token
        total += (first + L) * n // 2          # sum of p + 1 over the n new tokens
    return 4 * D * Hq * total


def bench_prefill(args):
    """Paged prefill of a batch of chat prompts (U[100, 2000] tokens, 32 heads
    of 128 dims, B = 16): per step, every prompt token's slot and K/V store
    (pa_append_kv) and causal prefill attention through the block
    tables (pa_prefill)."""
    import torch
    import paged_kv_cache_151_amd as pa
    import workloads as W
    torch.cuda.set_device(0)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    t0 = time.time()
    c = W.chat_prefill(S=args.prompts)
    kp, vp = dev(c.k_pool), dev(c.v_pool)
    tables, lens, qs = dev(c.block_tables), dev(c.context_lens), dev(c.query_start)
    q = dev(c.query)
    rng = np.random.default_rng(c.seed + 7)
    k_new = dev(W.f16_normal(rng, (c.T, c.Hkv, c.D)))
    v_new = dev(W.f16_normal(rng, (c.T, c.Hkv, c.D)))
    seq = dev(np.concatenate([np.full(n, s, np.int32) for s, n in enumerate(c.new_lens)]))
    pos = dev(np.concatenate([np.arange(L - n, L, dtype=np.int32)
                              for n, L in zip(c.new_lens, c.context_lens)]))
    slots = torch.empty(c.T, dtype=torch.int64, device="cuda")
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    flops = prefill_flops(c.new_lens, c.context_lens, c.Hq, c.D)
    log(f"setup {time.time() - t0:.1f}s: {c.name}, T={c.T}, NB={c.NB}, {flops / 1e9:.1f} GFLOP")

    def step(ev=None):
        pa.pa_append_kv(k_new, v_new, kp, vp, tables, seq_ids=seq, positions=pos, slot_mapping=slots)
        if ev is not None:
            ev[0].record(stream)
        pa.pa_prefill(q, kp, vp, tables, lens, qs, c.max_query_len, c.scale, out=out)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for e in ev:
        step(e)
    torch.cuda.synchronize()
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    tflops_step = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (launch_ms * 1e-3) / 1e12
    if args.copy_reference_mb > 0:
        copy_reference(args.copy_reference_mb)
    cpu = None if args.no_cpu_baseline else cpu_baseline_prefill(c, flops)
    print(json.dumps({
        "metric": "paged-prefill attention TFLOP/s (% of fp16 MFMA peak) + prompt tokens/s",
        "value": round(tflops_step, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "accumulate": "f32",
        "data": "synthetic", "prompt_tokens_per_s": round(c.T / (ms_per_step * 1e-3), 1),
        "config": {"workload": f"chat prefill: {c.S} prompts U[100,2000] tokens, nothing cached, "
                               f"32 heads x 128 dims fp16, B=16", "prompts": c.S,
                   "prompt_tokens": c.T, "max_prompt": c.max_query_len, "pool_blocks": c.NB,
                   "flops_per_step": int(flops)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": prefill_measured_traffic() if args.prompts == 16 else None,
                     "kernel": "pa_prefill (one launch per step)",
                     "avg_launch_us": round(launch_ms * 1e3, 2), "flops_per_launch": int(flops)},
        "cpu_baseline": cpu}), flush=True)


def cpu_baseline_prefill(c, flops_total, rows=48):
    """Oracle attention (fp64, numpy) for `rows` evenly spaced new tokens of every
    prompt, every head, over the keys each one sees; rate = their flops / time."""
    import oracle
    t_total, f_total = 0.0, 0
    group = c.Hq // c.Hkv
    for s in range(c.S):
        L, n, q0 = int(c.context_lens[s]), int(c.new_lens[s]), int(c.query_start[s])
        if n == 0:
            continue
        t = time.perf_counter()
        K = oracle.gather(c.k_pool, c.block_tables[s], L, c.B)
        V = oracle.gather(c.v_pool, c.block_tables[s], L, c.B)
        for j in np.linspace(0, n - 1, rows).astype(int):
            p = L - n + int(j)
            for h in range(c.Hq):
                oracle.attend(c.query[q0 + j, h], K[h // group, :p + 1], V[h // group, :p + 1], c.scale)
            f_total += 4 * c.D * c.Hq * (p + 1)
        t_total += time.perf_counter() - t
    return {"value": round(f_total / t_total / 1e12, 6), "unit": "TFLOP/s",
            "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"oracle attention of {rows} evenly spaced new tokens per prompt x {c.Hq} heads "
                      f"({c.S * rows * c.Hq} rows, {f_total / 1e9:.2f} GFLOP), {t_total:.1f} s"}


def bench_prefix_prefill(args):
    """The shared-prefix flow as prefill (grouped heads 32/8, B = 16): 64
    sequences share a cached 500-token prompt; per step, one pa_copy_blocks
    call (each sequence's private copy of the partly filled prompt block), the
    suffix tokens' slots and K/V stores, and pa_prefill over the 64 suffixes
    (U[50, 500] new tokens each, attending to the prompt and their own tokens)."""
    import torch
    import oracle
    import paged_kv_cache_151_amd as pa
    import workloads as W
    torch.cuda.set_device(0)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    t0 = time.time()
    d = W.prefix_prefill()
    S, B, NB = d["S"], d["B"], d["NB"]
    seq = np.concatenate([np.full(n, s, np.int32) for s, n in enumerate(d["new_lens"])])
    pos = np.concatenate([np.arange(d["prefix_len"], L, dtype=np.int32) for L in d["context_lens"]])
    kp, vp = dev(d["k_pool"]), dev(d["v_pool"])
    tables, lens, qs = dev(d["tables"]), dev(d["context_lens"]), dev(d["query_start"])
    pairs, q = dev(d["copy_pairs"]), dev(d["prefill_query"])
    ks, vs = dev(np.concatenate(d["suffix_k"])), dev(np.concatenate(d["suffix_v"]))
    seq_d, pos_d = dev(seq), dev(pos)
    slots = torch.empty(len(seq), dtype=torch.int64, device="cuda")
    out = torch.empty_like(q)
    maxq = int(d["new_lens"].max())
    stream = torch.cuda.current_stream()
    flops = prefill_flops(d["new_lens"], d["context_lens"], d["Hq"], d["D"])
    log(f"setup {time.time() - t0:.1f}s: prefix prefill, T={len(seq)}, NB={NB}, {flops / 1e9:.1f} GFLOP")

    def step(ev=None):
        pa.pa_copy_blocks(kp, vp, pairs)
        pa.pa_append_kv(ks, vs, kp, vp, tables, seq_ids=seq_d, positions=pos_d, slot_mapping=slots)
        if ev is not None:
            ev[0].record(stream)
        pa.pa_prefill(q, kp, vp, tables, lens, qs, maxq, d["scale"], out=out)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for e in ev:
        step(e)
    torch.cuda.synchronize()
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    achieved = flops / (launch_ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        rk, rv = oracle.copy_blocks(d["k_pool"], d["v_pool"], d["copy_pairs"])
        rk, rv = oracle.write_kv(rk, rv, np.concatenate(d["suffix_k"]), np.concatenate(d["suffix_v"]),
                                 oracle.token_slots(d["tables"], seq, pos, B, NB))
        c = W.PrefillCase(name="prefix_prefill", seed=4, S=S, Hq=d["Hq"], Hkv=d["Hkv"], D=d["D"], B=B,
                          NB=NB, context_lens=d["context_lens"], new_lens=d["new_lens"],
                          query_start=d["query_start"], block_tables=d["tables"],
                          query=d["prefill_query"], k_pool=rk, v_pool=rv, scale=d["scale"])
        cpu = cpu_baseline_prefill(c, flops, rows=12)
    print(json.dumps({
        "metric": "paged-prefill attention TFLOP/s (% of fp16 MFMA peak) + prompt tokens/s",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 1), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "accumulate": "f32", "data": "synthetic",
        "prompt_tokens_per_s": round(len(seq) / (ms_per_step * 1e-3), 1),
        "config": {"workload": "prefix prefill: 64 suffixes of U[50,500] tokens after a shared cached "
                               "500-token prompt, 32 query / 8 KV heads x 128 dims fp16, B=16",
                   "prompts": S, "new_tokens": len(seq), "max_new": maxq, "pool_blocks": NB,
                   "flops_per_step": int(flops)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "pa_prefill (one launch per step)",
                     "avg_launch_us": round(launch_ms * 1e3, 2), "flops_per_launch": int(flops)},
        "cpu_baseline": cpu}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path has no cross-GPU step "
              "(sequences and KV heads shard with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "prefill":
        bench_prefill(args)
        return
    if args.workload == "prefix_prefill":
        bench_prefix_prefill(args)
        return
    if args.workload == "block_manager":
        bench_block_manager(args)
        return
    if args.workload == "swap":
        bench_swap(args)
        return

    import torch
    import paged_kv_cache_151_amd as pa
    import workloads as W

    torch.cuda.set_device(0)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    t0 = time.time()
    if args.workload == "chat":
        steps_inputs, desc, extra = build_chat(args, dev)
    elif args.workload == "7b":
        steps_inputs, desc, extra = build_single(
            args, dev, W.seven_b_single_layer(),
            "7B-class single layer, batch 8, lengths U[50,900) (seed 7), 32 heads, B=16")
    elif args.workload == "long_context":
        c = W.long_context(with_pools=False)
        kp, vp = W.device_pools(c.NB, c.Hkv, c.B, c.D, seed=c.seed * 1000)
        c.k_pool, c.v_pool = kp, vp
        steps_inputs, desc, extra = build_single(
            args, lambda x: x if hasattr(x, "is_cuda") else dev(x), c,
            "long context, batch 16 x 4096 tokens, 32 heads, B=32")
    elif args.workload == "tiny":
        steps_inputs, desc, extra = build_single(
            args, dev, W.tiny_worked_example(),
            "tiny worked example, 2 sequences (40, 48 tokens), 4 heads, B=16")
    else:
        steps_inputs, desc, extra = build_shared_prefix(args, dev, pa)
    torch.cuda.synchronize()
    c0 = steps_inputs[0][0]["case"]
    S = c0.S
    log(f"setup {time.time() - t0:.1f}s: {desc}; {len(steps_inputs)} input set(s) x "
        f"{len(steps_inputs[0])} layer(s), NB={c0.NB}")

    maxL = max(ly["case"].max_context_len for ly in steps_inputs[0])
    P = pa.pa_decode_partition_size(S, c0.Hq, c0.Hkv, c0.B, maxL, args.partition_size)
    ws_bytes = pa.pa_decode_workspace_bytes(S, c0.Hq, c0.Hkv, c0.D, c0.B, maxL, P)
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    out = torch.empty((S, c0.Hq, c0.D), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(k, events=None):
        for i, ly in enumerate(steps_inputs[k % len(steps_inputs)]):
            c = ly["case"]
            pa.pa_append_kv(ly["k_new"], ly["v_new"], ly["kp"], ly["vp"], ly["tables"],
                            context_lens=ly["lens"], slot_mapping=ly["slots"])
            if events is not None:
                events[i][0].record(stream)
            pa.pa_decode(ly["q"], ly["kp"], ly["vp"], ly["tables"], ly["lens"], maxL, c.scale,
                         partition_size=P, out=out, workspace=workspace)
            if events is not None:
                events[i][1].record(stream)

    graphs = None
    if args.graph:
        # one graph per input set, captured after an eager run of every set
        for k in range(len(steps_inputs)):
            step(k)
        torch.cuda.synchronize()
        graphs = []
        for k in range(len(steps_inputs)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(k)
            graphs.append(g)
        torch.cuda.synchronize()
    run_step = (lambda k: graphs[k % len(graphs)].replay()) if graphs else step

    for k in range(args.warmup):
        run_step(k)
    torch.cuda.synchronize()

    # timed region: K whole steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(args.steps):
        run_step(k)
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps

    # decode-call durations: events around every pa_decode of further steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in steps_inputs[0]] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(k, ev[k])
    torch.cuda.synchronize()
    decode_ms = np.array([[a.elapsed_time(b) for a, b in row] for row in ev])
    decode_avg_ms = float(decode_ms.mean())

    kv_bytes_layer = [ly["case"].kv_bytes() for ly in steps_inputs[0]]
    kv_bytes_step = float(sum(kv_bytes_layer))
    gbs = kv_bytes_step / (ms_per_step * 1e-3) / 1e9
    tok_s = S / (ms_per_step * 1e-3)
    achieved = float(np.mean(kv_bytes_layer)) / (decode_avg_ms * 1e-3) / 1e9

    cow = time_copy_on_write(pa, extra) if "copy" in extra else None
    stream = stream_ceiling(pa, steps_inputs) if args.workload in ("chat", "long_context") else None

    if args.copy_reference_mb > 0:
        copy_reference(args.copy_reference_mb)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(steps_inputs[0], args.cpu_sample_layers, kv_bytes_step,
                           len(steps_inputs[0]))

    config = {
        "workload": desc,
        "batch": S, "layers": len(steps_inputs[0]), "heads_q": c0.Hq, "heads_kv": c0.Hkv,
        "head_dim": c0.D, "block_size": c0.B, "pool_blocks_per_layer": c0.NB,
        "tokens_per_layer": int(c0.context_lens.sum()), "max_context": maxL, "partition_size": P,
        "kv_bytes_per_step": int(kv_bytes_step),
        "launch": "HIP graph replay per step" if graphs else "eager calls",
    }
    if "replicas" in extra:
        config["input_replicas_rotated"] = extra["replicas"]
    res = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "accumulate": "f32",
        "data": "synthetic",
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(tok_s, 1),
        "config": config,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (measured_traffic() if args.workload == "chat" and args.layers == 32
                        and args.block_size == 16 and not args.contiguous
                        and (args.q_heads, args.kv_heads) == (32, 32) else None),
            "kernel": "pa_decode call (partition + reduce kernels), average per layer",
            "avg_launch_us": round(decode_avg_ms * 1e3, 2),
            "median_launch_us": round(float(np.median(decode_ms)) * 1e3, 2),
            "bytes_per_launch": int(np.mean(kv_bytes_layer)),
            "other_bytes_per_launch": other_bytes(c0, P),
        },
        "cpu_baseline": cpu,
    }
    if cow is not None:
        res["copy_on_write"] = cow
    if stream is not None:
        res["stream_read"] = {"GBs": stream["GBs"], "workgroups": stream["workgroups"],
                              "decode_vs_stream": round(achieved / stream["GBs"], 4),
                              "what": "pa_stream_read: one linear pass over this run's K/V pools "
                                      "(8 16-byte loads in flight per lane, nt + sc1), best of 6 "
                                      "launch shapes (512 to 16,384 workgroups of 256 threads)"}
    print(json.dumps(res), flush=True)


def other_bytes(c, P):
    """Bytes one pa_decode call moves besides the counted K/V of valid tokens:
    the rest of each sequence's last block (touched by nothing but counted by
    a whole-block reader), query and output, table entries and lengths read,
    and the partials written and read back across partitions."""
    L = c.context_lens.astype(np.int64)
    blocks = -(-L // c.B)
    row = c.Hkv * c.D * 2 * 2                     # K and V bytes of one token, all KV heads
    nparts = -(-L // P)
    G = c.Hq // c.Hkv
    parts = int(-(-int(L.max()) // P))
    even = parts > 1 and c.S <= 1024 and (G >= 4 or c.S * c.Hkv * parts > 2048)
    if even:
        # even split: runs of q units over the (KV head, sequence, unit)
        # order, one per workgroup of the grid (2 per compute unit, 6 for two
        # heads per KV head)
        n = -(-L // 16)
        N = int(n.sum())
        resident = 1536 if G == 2 else 512
        grid = min(resident, -(-c.S * c.Hkv * parts // 8) * 8)
        q = max(-(-N * c.Hkv // grid), P // 16)
        first = (np.arange(c.Hkv)[:, None] * N + (np.cumsum(n) - n)[None, :])
        pieces = (first + n[None, :] - 1) // q - first // q + 1
        pieces = pieces[n[None, :].repeat(c.Hkv, 0) > 0]
        partial_rows = int(pieces[pieces > 1].sum()) * G
    else:
        partial_rows = int(nparts[nparts > 1].sum()) * c.Hq
    return {
        "kv_unread_tail_of_last_blocks": int((blocks * c.B - L).sum() * row),
        "query_and_output": int(2 * c.S * c.Hq * c.D * 2),
        "tables_and_lengths": int(blocks.sum() * 4 + c.S * 4),
        # a piece's row: its normalised result in fp16 and its maximum and sum in fp32
        "workspace_partials_written_and_read": int(2 * partial_rows * (c.D * 2 + 8)),
    }


def stream_ceiling(pa, steps_inputs):
    """Practical read ceiling on this GPU in this run: pa_stream_read over the
    workload's own pools, rotated so that no pass is served by the caches."""
    import torch
    bufs, total = [], 0
    for ly in steps_inputs[0]:
        for t in (ly["kp"], ly["vp"]):
            if t.numel() * t.element_size() >= (256 << 20):
                bufs.append(t)
                total += t.numel() * t.element_size()
        if total >= (1536 << 20):
            break
    if total < (1024 << 20):
        return None
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    best = None
    for wg in (512, 1024, 2048, 4096, 8192, 16384):   # 2 to 64 workgroups of 4 waves per CU
        for b in bufs:
            pa.pa_stream_read(b, sink, wg)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 2 * len(bufs)
        nbytes = 0
        e0.record()
        for r in range(reps):
            b = bufs[r % len(bufs)]
            pa.pa_stream_read(b, sink, wg)
            nbytes += b.numel() * b.element_size()
        e1.record()
        torch.cuda.synchronize()
        gbs = nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
        if best is None or gbs > best["GBs"]:
            best = {"GBs": round(gbs, 1), "workgroups": wg}
    return best


def cpu_baseline(layers, n_sample, kv_bytes_step, n_layers):
    """Oracle decode (gather through the table, fp64 attention) on the host for
    `n_sample` evenly spaced layers (every layer when n_sample >= the step's
    layers), on the same inputs the GPU saw. The step's oracle time is the
    mean layer time times the number of layers; its relative standard error
    over the sampled layers is reported with it."""
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    n_sample = max(1, min(n_sample, len(layers)))
    picks = sorted({int(round(x)) for x in np.linspace(0, len(layers) - 1, n_sample)})
    per_layer = []
    tokens = 0
    for i in picks:
        ly = layers[i]
        c = ly["case"]
        used = np.unique(c.block_tables[c.block_tables >= 0])
        idx = torch.from_numpy(used.astype(np.int64)).cuda()
        kb = ly["kp"][idx].cpu().numpy()
        vb = ly["vp"][idx].cpu().numpy()
        remap = np.full(c.NB, -1, np.int64)
        remap[used] = np.arange(len(used))
        tables = np.where(c.block_tables >= 0, remap[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
        t = time.perf_counter()
        oracle.decode(c.query, kb, vb, tables, c.context_lens, c.scale)
        per_layer.append(time.perf_counter() - t)
        tokens += int(c.context_lens.sum())
        del kb, vb
        log(f"cpu baseline: layer {i} {per_layer[-1]:.2f} s")
    secs = float(np.sum(per_layer))
    mean = secs / len(per_layer)
    if len(per_layer) == len(layers):
        rel_err = 0.0
    elif len(per_layer) > 1:
        rel_err = float(np.std(per_layer, ddof=1) / np.sqrt(len(per_layer)) / mean)
    else:
        rel_err = None
    step_s = mean * n_layers
    kv_layer = kv_bytes_step / n_layers
    S = layers[0]["case"].S
    return {
        "value": round(kv_layer / mean / 1e9, 4),
        "unit": "GB/s",
        "cores": len(os.sched_getaffinity(0)),
        "blas_threads": blas_threads,
        "kind": "oracle",
        "decode_tokens_per_s": round(S / step_s, 4),
        "step_s": round(step_s, 2),
        "step_s_rel_std_err": None if rel_err is None else round(rel_err, 4),
        "layers_timed": picks,
        "per_layer_s": [round(x, 3) for x in per_layer],
        "sample": f"oracle decode of {len(picks)} of {n_layers} layer(s), evenly spaced (all {S} "
                  f"sequences, {tokens} cached tokens x {layers[0]['case'].Hq} query heads), "
                  f"{secs:.1f} s; the {n_layers}-layer step time is the mean layer time x "
                  f"{n_layers}" + ("" if len(picks) == n_layers else
                                   f", relative standard error {rel_err}"),
    }


if __name__ == "__main__":
    main()
