import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture
def golden():
    return load_golden


@pytest.fixture(autouse=True)
def _bounds_audit(request):
    """With PA_TEST_BOUNDS=1 and the bounds-checked build loaded as the
    library (libpa_debug.so in place of libpa.so), every GPU test must end with
    no refused access at any check site. The release build has no such checks:
    there each counted access would have left its buffer."""
    yield
    if os.environ.get("PA_TEST_BOUNDS") != "1" or request.node.get_closest_marker("gpu") is None:
        return
    import torch

    import paged_kv_cache_151_amd as pa
    torch.cuda.synchronize()
    v = pa.pa_debug_bounds_violations()
    assert v is not None, "PA_TEST_BOUNDS=1 needs the bounds-checked library in use"
    assert not any(v.values()), f"{request.node.nodeid}: refused accesses {v}"
