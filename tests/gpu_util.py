"""Helpers for the GPU parity tests: device transfer, the attention tolerance,
and loading the HIP binding (which fails loudly when libpa.so is missing)."""
import sys

import numpy as np
import pytest

# |gpu - ref| <= ABS + REL * |ref| elementwise, for fp16-in / fp32-accumulate
# attention against the fp64 oracle
TOL_ABS = 2e-3
TOL_REL = 1e-2


def pa_module():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import paged_kv_cache_151_amd as pa
    return pa


def say(*msg):
    """Name the case on stdout before GPU work, so a failing run shows where it was."""
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def u16(a):
    return np.ascontiguousarray(a).view(np.uint16)


def assert_attention_close(got_f16, ref64, what=""):
    got = np.asarray(got_f16, dtype=np.float64)
    assert got.shape == ref64.shape, (got.shape, ref64.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    diff = np.abs(got - ref64)
    bound = TOL_ABS + TOL_REL * np.abs(ref64)
    bad = diff > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(diff - bound), diff.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {idx}: "
            f"got {got[idx]:.6g} ref {ref64[idx]:.6g} (max abs err {diff.max():.3g})")
    return float(diff.max())
