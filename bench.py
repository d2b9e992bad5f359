"""Benchmark: paged decode on the batch-128 chat workload, one MI355X.

Workload: 128 sequences, context = prompt U[100, 2000] + generated U[50, 500]
tokens, 32 layers, each with its own K/V block pool (32 KV heads, head dim 128,
fp16, blocks of 16 tokens, 1.25x pool, shuffled physical ids). One step is one
decode step of the whole model's attention cache path: per layer, the new
token's slot (pa_slot_mapping), its K/V store (pa_write_kv) and paged decode
attention (pa_decode). Inputs are synthetic (seeded) and resident in HBM before
the timed region.

Prints one JSON line. `value` is KV bytes read per step (valid tokens x 32
heads x 128 x K and V x 2 B, summed over layers) divided by the step time.
`roofline` prices the decode call (partition + reduce kernels), timed with HIP
events on the stream it runs on, against 8 TB/s. `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
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


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--cpu-sample-layers", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-reference-mb", type=int, default=0,
                    help="after timing, run one pa_copy_blocks moving this many MiB per pool "
                         "(a copy of known size for scaling traffic counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pa_decode_chat_b128_traffic.json")
DECODE_SOURCES = [os.path.join(ROOT, "paged_kv_cache_151_amd", "csrc", f)
                  for f in ("decode.hip", "pa_internal.h")]


def decode_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode launch from the committed counter summary, or None
    when the decode kernel's source changed after the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("decode_source_sha256") != decode_source_hash():
        return None
    return t.get("traffic_bytes_per_launch")


def copy_reference(pa, mb):
    """One pa_copy_blocks call over a scratch pool: reads and writes exactly
    mb MiB in each of two pools (K and V)."""
    import torch
    blk = 32 * 16 * 128 * 2                       # bytes of one block of one pool
    n = max(1, (mb << 20) // blk)
    kp = torch.empty((2 * n, 32, 16, 128), dtype=torch.float16, device="cuda")
    vp = torch.empty_like(kp)
    pairs = torch.stack([torch.arange(n), torch.arange(n) + n], 1).to(torch.int32).cuda()
    torch.cuda.synchronize()
    pa.pa_copy_blocks(kp, vp, pairs)
    torch.cuda.synchronize()
    log(f"copy reference: {n} blocks x {blk} B per pool, {2 * n * blk} B read, same written")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path has no cross-GPU step "
              "(sequences and KV heads shard with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.layers != 32:
        log("note: --layers != 32 is a reduced workload; the JSON line says so")

    import torch
    import paged_kv_cache_151_amd as pa
    import workloads as W

    torch.cuda.set_device(0)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    lengths = W.chat_lengths()
    S = len(lengths)
    layers = []
    t0 = time.time()
    for layer in range(args.layers):
        c = W.chat_layer(layer, lengths=lengths)
        kp, vp = W.device_pools(c.NB, c.Hkv, c.B, c.D, seed=W.chat_pool_seed(layer))
        layers.append(dict(case=c, kp=kp, vp=vp, tables=dev(c.block_tables),
                           lens=dev(c.context_lens), q=dev(c.query), k_new=dev(c.key_new),
                           v_new=dev(c.value_new),
                           slots=torch.empty(S, dtype=torch.int64, device="cuda")))
    torch.cuda.synchronize()
    c0 = layers[0]["case"]
    pool_gb = 2 * c0.NB * c0.Hkv * c0.B * c0.D * 2 / 1e9
    log(f"setup {time.time() - t0:.1f}s: {args.layers} layers, NB={c0.NB}, "
        f"K+V pools {pool_gb:.2f} GB per layer")
    maxL = c0.max_context_len
    P = pa.pa_decode_partition_size(S, c0.Hkv, c0.B, maxL, args.partition_size)
    ws_bytes = pa.pa_decode_workspace_bytes(S, c0.Hq, c0.Hkv, c0.D, c0.B, maxL, P)
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    out = torch.empty((S, c0.Hq, c0.D), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(events=None):
        for i, ly in enumerate(layers):
            c = ly["case"]
            pa.pa_slot_mapping(ly["tables"], c.B, c.NB, context_lens=ly["lens"], out=ly["slots"])
            pa.pa_write_kv(ly["k_new"], ly["v_new"], ly["kp"], ly["vp"], ly["slots"])
            if events is not None:
                events[i][0].record(stream)
            pa.pa_decode(ly["q"], ly["kp"], ly["vp"], ly["tables"], ly["lens"], maxL, c.scale,
                         partition_size=P, out=out, workspace=workspace)
            if events is not None:
                events[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps

    # decode-call durations: events around every pa_decode of further steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in layers] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    decode_ms = np.array([[a.elapsed_time(b) for a, b in row] for row in ev])
    decode_avg_ms = float(decode_ms.mean())

    kv_bytes_layer = [ly["case"].kv_bytes() for ly in layers]
    kv_bytes_step = float(sum(kv_bytes_layer))
    gbs = kv_bytes_step / (ms_per_step * 1e-3) / 1e9
    tok_s = S / (ms_per_step * 1e-3)
    achieved = float(np.mean(kv_bytes_layer)) / (decode_avg_ms * 1e-3) / 1e9

    if args.copy_reference_mb > 0:
        copy_reference(pa, args.copy_reference_mb)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(layers, args.cpu_sample_layers, kv_bytes_step, args.layers)

    res = {
        "metric": "paged-decode KV-read GB/s (% of HBM peak) + decode tokens/s, batch 128",
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
        "config": {
            "workload": "chat decode, batch 128, 32 layers (prompt U[100,2000] + generated U[50,500])",
            "batch": S, "layers": args.layers, "heads_q": c0.Hq, "heads_kv": c0.Hkv,
            "head_dim": c0.D, "block_size": c0.B, "pool_blocks_per_layer": c0.NB,
            "tokens": int(lengths.sum()), "max_context": maxL, "partition_size": P,
            "kv_bytes_per_step": int(kv_bytes_step),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "kernel": "pa_decode (partition + reduce), average per layer call",
            "avg_launch_us": round(decode_avg_ms * 1e3, 2),
            "bytes_per_launch": int(np.mean(kv_bytes_layer)),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def cpu_baseline(layers, n_sample, kv_bytes_step, n_layers):
    """Oracle decode (gather through the table, fp64 attention) on the host for
    the first `n_sample` layers, on the same inputs the GPU saw."""
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    n_sample = max(1, min(n_sample, len(layers)))
    secs = 0.0
    tokens = 0
    for ly in layers[:n_sample]:
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
        secs += time.perf_counter() - t
        tokens += int(c.context_lens.sum())
        del kb, vb
    per_layer = secs / n_sample
    kv_layer = kv_bytes_step / n_layers
    return {
        "value": round(kv_layer / per_layer / 1e9, 4),
        "unit": "GB/s",
        "cores": len(os.sched_getaffinity(0)),
        "blas_threads": blas_threads,
        "kind": "oracle",
        "decode_tokens_per_s": round(layers[0]["case"].S / (per_layer * n_layers), 4),
        "sample": f"oracle decode of {n_sample} of {n_layers} layers (all 128 sequences, "
                  f"{tokens} cached tokens x 32 heads), {secs:.1f} s; tokens/s extrapolated "
                  f"to the 32-layer step",
    }


if __name__ == "__main__":
    main()
