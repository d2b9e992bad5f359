"""The read-bandwidth probe (a measurement utility, not part of the attention
path) runs cleanly and writes nothing for ordinary data."""
import pytest

from gpu_util import pa_module, say

pytestmark = pytest.mark.gpu


def test_stream_read_runs_and_leaves_sink_alone():
    import torch
    pa = pa_module()
    say("pa_stream_read over 64 MiB of zeros and of ones")
    for fill in (0, 1):
        buf = torch.full((32 << 20,), fill, dtype=torch.float16, device="cuda")
        sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
        for wg in (1, 64, 4096):
            pa.pa_stream_read(buf, sink, wg)
        pa.pa_stream_read(buf, sink, 256, nbytes=4096 + 16)   # a partial pass
        torch.cuda.synchronize()
        assert sink.cpu().tolist() == [7, 7, 7, 7]
