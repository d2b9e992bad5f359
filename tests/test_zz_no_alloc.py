"""pa_decode_static, the decode entry point that allocates nothing (its
partials live in a per-GPU scratch array inside the library), against
pa_decode with a caller workspace: bit-identical outputs on two calls in a row,
the second smaller than the first, both within the tolerance of the oracle;
and the refusal of a call whose partials exceed the array."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_attention_close, dev, host, pa_module, say, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return pa_module()


def _run_both(pa, c, P):
    import torch
    tables, lens, q = dev(c.block_tables), dev(c.context_lens), dev(c.query)
    kp, vp = dev(c.k_pool), dev(c.v_pool)
    ws = pa.pa_decode_workspace_bytes(c.S, c.Hq, c.Hkv, c.D, c.B, c.max_context_len, P)
    assert 0 < ws <= pa.pa_decode_static_scratch_bytes()
    ref_out = pa.pa_decode(q, kp, vp, tables, lens, c.max_context_len, c.scale, partition_size=P)
    out = torch.empty_like(q)
    pa.pa_decode_static(q, kp, vp, tables, lens, c.max_context_len, c.scale, partition_size=P,
                        out=out)
    return host(out), host(ref_out)


def test_static_scratch_matches_workspace_on_two_calls_the_second_smaller(pa):
    big = W.make_case("static_big", 9901, [3000, 17, 1, 2049, 1200, 777, 0, 2500], Hq=32, Hkv=8,
                      B=16)
    small = W.make_case("static_small", 9902, [300, 45, 129], Hq=4, Hkv=4, B=16)
    for c, P in ((big, 256), (small, 64)):
        say(c.name, f"S={c.S} Hq={c.Hq} Hkv={c.Hkv} P={P}")
        got, want = _run_both(pa, c, P)
        assert np.array_equal(u16(got), u16(want)), f"{c.name}: differs from pa_decode"
        ref = oracle.decode(c.query, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale)
        assert_attention_close(got, ref, c.name)


def test_static_scratch_refuses_partials_beyond_its_size(pa):
    import torch
    c = W.make_case("static_refuse", 9903, [40, 48], Hq=4, Hkv=4, B=16)
    q = dev(c.query)
    # sizes (not contents) make the partials exceed the array: 4096 sequences
    # x 64 heads x 2 partitions of 16 tokens need 4096 * 64 * 2 * 130 * 4 bytes
    S, H = 4096, 64
    qq = torch.zeros((S, H, c.D), dtype=torch.float16, device="cuda")
    pool = torch.zeros((16, H, 16, c.D), dtype=torch.float16, device="cuda")
    tables = torch.zeros((S, 2), dtype=torch.int32, device="cuda")
    lens = torch.full((S,), 32, dtype=torch.int32, device="cuda")
    need = pa.pa_decode_workspace_bytes(S, H, H, c.D, 16, 32, 16)
    assert need > pa.pa_decode_static_scratch_bytes()
    with pytest.raises(pa.PaError, match="PA_ERR_WORKSPACE"):
        pa.pa_decode_static(qq, pool, pool, tables, lens, 32, c.scale, partition_size=16)
    del q
