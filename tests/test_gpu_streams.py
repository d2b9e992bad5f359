"""Calls on two streams at once. Every call is asynchronous on the stream it
is given (torch's current stream in the binding) and the kernels keep no state
between calls apart from a call's own workspace, so decode and prefill
launched on two streams in turn, each with its own buffers, give exactly the
results of the same calls made one after another."""
import numpy as np
import pytest

import workloads as W
from gpu_util import dev, host, pa_module, say, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return pa_module()


def test_decode_and_prefill_on_two_streams_match_serial_calls(pa):
    import torch
    cases = [W.make_case("streams_a", 8200, [900, 33, 2100, 400], Hq=32, Hkv=8, B=16),
             W.make_case("streams_b", 8201, [1500, 64, 7, 1200, 300], Hq=16, Hkv=16, B=32)]
    pf = W.make_prefill_case("streams_prefill", 8202, [120, 40, 300], [0, 500, 64], Hq=8, Hkv=2,
                             B=16)
    say("two streams: grouped and MHA decode, prefill")
    P = 256
    inputs = []
    for c in cases:
        ws = torch.empty(max(pa.pa_decode_workspace_bytes(c.S, c.Hq, c.Hkv, c.D, c.B,
                                                          c.max_context_len, P), 16),
                         dtype=torch.uint8, device="cuda")
        inputs.append((c, (dev(c.query), dev(c.k_pool), dev(c.v_pool), dev(c.block_tables),
                           dev(c.context_lens)), ws))
    pf_args = (dev(pf.query), dev(pf.k_pool), dev(pf.v_pool), dev(pf.block_tables),
               dev(pf.context_lens), dev(pf.query_start))

    def decode(i, out, stream=None):
        c, args, ws = inputs[i]
        return pa.pa_decode(*args, c.max_context_len, c.scale, partition_size=P, out=out,
                            workspace=ws, stream=stream)

    # serial reference, one call after another on the current stream
    serial = [host(decode(i, torch.empty_like(inputs[i][1][0]))).copy() for i in range(2)]
    serial_pf = host(pa.pa_prefill(*pf_args, pf.max_query_len, pf.scale)).copy()

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    outs = [torch.empty_like(inputs[i][1][0]) for i in range(2)]
    out_pf = torch.empty_like(pf_args[0])
    torch.cuda.synchronize()
    for rep in range(5):
        for o in outs + [out_pf]:
            o.fill_(3.0)
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            decode(0, outs[0])
            pa.pa_prefill(*pf_args, pf.max_query_len, pf.scale, out=out_pf)
        with torch.cuda.stream(s2):
            decode(1, outs[1])
        with torch.cuda.stream(s2):
            decode(1, outs[1])   # again, overlapping the first stream's work
        torch.cuda.synchronize()
        for i in range(2):
            assert np.array_equal(u16(host(outs[i])), u16(serial[i])), f"decode {i}, round {rep}"
        assert np.array_equal(u16(host(out_pf)), u16(serial_pf)), f"prefill, round {rep}"
