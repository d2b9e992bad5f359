"""Decode and prefill steps captured in a HIP graph (torch.cuda.CUDAGraph around
the binding's calls, which launch on torch's current stream) replay bit for bit
like the same calls run eagerly. Each replay follows eager work on the same
buffers (the output is cleared and the pool entries the step writes are
overwritten), so a replay that reused stale state would show."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_attention_close, dev, host, pa_module, say, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return pa_module()


def _grouped_case():
    # groups of 4 over several partitions: the even split, with its piece
    # counts and partials in the workspace for the reduce kernel
    return W.make_case("graph_grouped", 8100, [700, 1500, 33, 900, 0, 260, 1023, 64],
                       Hq=32, Hkv=8, B=16)


@pytest.mark.parametrize("which", ["7b", "grouped"])
def test_decode_step_replays_bit_identical(pa, which):
    import torch
    c = W.seven_b_single_layer() if which == "7b" else _grouped_case()
    say(c.name, "decode step in a graph")
    kp, vp = dev(c.k_pool), dev(c.v_pool)
    tables, lens = dev(c.block_tables), dev(c.context_lens)
    q, k_new, v_new = dev(c.query), dev(c.key_new), dev(c.value_new)
    P = 256   # several partitions: the partials, the reduce kernel and the workspace are in the graph
    ws = torch.empty(max(pa.pa_decode_workspace_bytes(c.S, c.Hq, c.Hkv, c.D, c.B,
                                                      c.max_context_len, P), 16),
                     dtype=torch.uint8, device="cuda")
    slots = torch.empty(c.S, dtype=torch.int64, device="cuda")
    out = torch.empty_like(q)

    def step():
        pa.pa_slot_mapping(tables, c.B, c.NB, context_lens=lens, out=slots)
        pa.pa_write_kv(k_new, v_new, kp, vp, slots)
        pa.pa_decode(q, kp, vp, tables, lens, c.max_context_len, c.scale, partition_size=P,
                     out=out, workspace=ws)

    step()
    eager = host(out).copy()
    ref = oracle.decode(c.query, *oracle.write_kv(c.k_pool, c.v_pool, c.key_new, c.value_new,
                                                  oracle.decode_slots(c.block_tables, c.context_lens,
                                                                      c.B, c.NB)),
                        c.block_tables, c.context_lens, c.scale)
    assert_attention_close(eager, ref, "eager decode")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        slots.fill_(-1)
        kp.view(-1)[:4096].zero_()            # unrelated eager writes to the pool between replays
        kp.view(-1)[:4096] = dev(c.k_pool).view(-1)[:4096]
        if r == 1:
            # an eager call on the same workspace between replays
            other = torch.empty_like(out)
            pa.pa_decode(q, kp, vp, tables, lens, c.max_context_len, c.scale, partition_size=P,
                         out=other, workspace=ws)
            assert np.array_equal(u16(host(other)), u16(eager))
            slots.fill_(-1)
        g.replay()
        got = host(out)
        assert np.array_equal(u16(got), u16(eager)), f"replay {r}"
        assert np.array_equal(host(slots), oracle.decode_slots(c.block_tables, c.context_lens, c.B, c.NB))


def test_prefill_step_replays_bit_identical(pa):
    import torch
    c = W.make_prefill_case("graph_prefill", 3900, [70, 200, 9], [30, 0, 300], Hq=8, Hkv=2, B=16)
    say(c.name, "prefill in a graph")
    kp, vp = dev(c.k_pool), dev(c.v_pool)
    args = (dev(c.query), kp, vp, dev(c.block_tables), dev(c.context_lens), dev(c.query_start))
    out = torch.empty_like(args[0])

    def step():
        pa.pa_prefill(*args, c.max_query_len, c.scale, out=out)

    step()
    eager = host(out).copy()
    assert_attention_close(eager, oracle.prefill(c.query, c.k_pool, c.v_pool, c.block_tables,
                                                 c.context_lens, c.query_start, c.scale),
                           "eager prefill")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(7.0)
        g.replay()
        assert np.array_equal(u16(host(out)), u16(eager)), f"replay {r}"


def test_static_decode_step_replays_bit_identical(pa):
    """pa_decode_static inside a captured graph: its partials live in the
    library's per-GPU scratch array, so the captured step allocates nothing.
    Before every replay an eager call on other inputs rewrites that scratch;
    each replay must still equal the eager step bit for bit (the kernels read
    only partials they wrote in the same call)."""
    import torch
    c = _grouped_case()
    other = W.make_case("graph_static_other", 8101, [1900, 5, 640], Hq=32, Hkv=8, B=16)
    say(c.name, "static decode step in a graph")
    P = 256
    for d in (c, other):
        need = pa.pa_decode_workspace_bytes(d.S, d.Hq, d.Hkv, d.D, d.B, d.max_context_len, P)
        assert 0 < need <= pa.pa_decode_static_scratch_bytes()
    kp, vp = dev(c.k_pool), dev(c.v_pool)
    tables, lens = dev(c.block_tables), dev(c.context_lens)
    q, k_new, v_new = dev(c.query), dev(c.key_new), dev(c.value_new)
    slots = torch.empty(c.S, dtype=torch.int64, device="cuda")
    out = torch.empty_like(q)

    def step():
        pa.pa_append_kv(k_new, v_new, kp, vp, tables, context_lens=lens, slot_mapping=slots)
        pa.pa_decode_static(q, kp, vp, tables, lens, c.max_context_len, c.scale, partition_size=P,
                            out=out)

    step()
    eager = host(out).copy()
    ref_slots = oracle.decode_slots(c.block_tables, c.context_lens, c.B, c.NB)
    ref = oracle.decode(c.query, *oracle.write_kv(c.k_pool, c.v_pool, c.key_new, c.value_new,
                                                  ref_slots),
                        c.block_tables, c.context_lens, c.scale)
    assert_attention_close(eager, ref, "eager static decode")
    o_args = (dev(other.query), dev(other.k_pool), dev(other.v_pool), dev(other.block_tables),
              dev(other.context_lens))
    o_out = torch.empty_like(o_args[0])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        slots.fill_(-1)
        pa.pa_decode_static(*o_args, other.max_context_len, other.scale, partition_size=P,
                            out=o_out)   # other partials into the same scratch
        torch.cuda.synchronize()
        g.replay()
        assert np.array_equal(u16(host(out)), u16(eager)), f"replay {r}"
        assert np.array_equal(host(slots), ref_slots)
