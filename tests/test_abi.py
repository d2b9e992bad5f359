"""The C-ABI library loads, exports every entry point the header declares, and
rejects bad arguments on the host before touching the GPU. No compute call
runs here: each call below fails validation before any HIP call."""
import ctypes
import os
import re

import pytest

from conftest import ROOT
from decode_rules import even_split

HEADER = os.path.join(ROOT, "include", "pa.h")
# PA_ABI_LIB: another build of the same sources (the host-sanitized one, for example)
LIB = os.environ.get("PA_ABI_LIB") or os.path.join(ROOT, "paged_kv_cache_151_amd", "libpa.so")

PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_ALIGN, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE = range(6)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libpa.so not built (run __graft_entry__.build())")
    l = ctypes.CDLL(LIB)
    l.pa_status_str.restype = ctypes.c_char_p
    l.pa_last_error.restype = ctypes.c_char_p
    l.pa_decode_workspace_bytes.restype = ctypes.c_size_t
    return l


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"pa_decode", "pa_write_kv", "pa_copy_blocks", "pa_slot_mapping", "pa_bm_create",
            "pa_bm_append_tokens", "pa_bm_fork", "pa_bm_release", "pa_bm_export"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


DEBUG_LIB = os.path.join(ROOT, "paged_kv_cache_151_amd", "libpa_debug.so")


def test_debug_library_exports_the_same_entry_points():
    # the bounds-checked build: same sources, same ABI
    if not os.path.exists(DEBUG_LIB):
        pytest.fail("libpa_debug.so not built (run __graft_entry__.build())")
    dbg = ctypes.CDLL(DEBUG_LIB)
    for n in declared_functions():
        assert hasattr(dbg, n), n
    dbg.pa_debug_bounds_site.restype = ctypes.c_char_p
    names = [dbg.pa_debug_bounds_site(i) for i in range(8)]
    assert names == [b"length", b"table", b"query", b"pool", b"out", b"partial", b"slot", b"pair"]
    assert dbg.pa_debug_bounds_site(8) is None and dbg.pa_debug_bounds_site(-1) is None


def test_release_library_has_no_bounds_counters(lib):
    counts = (ctypes.c_uint * 8)(*([7] * 8))
    assert lib.pa_debug_bounds_violations(counts, 8) == -1
    assert list(counts) == [7] * 8     # untouched
    assert lib.pa_debug_bounds_selftest() == -1


def test_status_strings(lib):
    assert lib.pa_status_str(0) == b"PA_OK"
    assert lib.pa_status_str(5) == b"PA_ERR_WORKSPACE"
    assert lib.pa_status_str(7) == b"PA_ERR_EXHAUSTED"
    assert lib.pa_status_str(8) == b"PA_ERR_STATE"
    assert lib.pa_status_str(99) == b"PA_ERR_UNKNOWN"
    assert lib.pa_version() >= 100


F = ctypes.c_float
Z = ctypes.c_size_t
FAKE = 0x1000          # an aligned non-null address; never dereferenced (validation fails first)


def decode(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, t=FAKE, l=FAKE, S=2, Hq=4, Hkv=4, D=128, B=16,
             NB=16, MB=3, maxL=48, scale=0.1, P=0, ws=None, wsb=0)
    a.update(kw)
    return lib.pa_decode(ctypes.c_void_p(a["out"]), ctypes.c_void_p(a["q"]), ctypes.c_void_p(a["k"]),
                         ctypes.c_void_p(a["v"]), ctypes.c_void_p(a["t"]), ctypes.c_void_p(a["l"]),
                         a["S"], a["Hq"], a["Hkv"], a["D"], a["B"], a["NB"], a["MB"], a["maxL"],
                         F(a["scale"]), a["P"], ctypes.c_void_p(a["ws"]), Z(a["wsb"]), None)


def test_decode_host_validation(lib):
    assert decode(lib, out=None) == PA_ERR_NULL
    assert b"null" in lib.pa_last_error()
    assert decode(lib, Hq=6, Hkv=4) == PA_ERR_SHAPE
    assert decode(lib, D=64) == PA_ERR_UNSUPPORTED
    assert decode(lib, B=24, NB=16, MB=2) == PA_ERR_UNSUPPORTED   # 8 and multiples of 16 only
    assert decode(lib, B=8, NB=16, MB=6, out=None) == PA_ERR_NULL   # B = 8 passes validation
    assert decode(lib, Hq=48, Hkv=4) == PA_ERR_UNSUPPORTED      # group of 12
    assert decode(lib, maxL=49) == PA_ERR_SHAPE                 # beyond MB * B
    assert decode(lib, P=24) == PA_ERR_SHAPE                    # not a multiple of 16
    assert decode(lib, B=40, NB=16, MB=2) == PA_ERR_UNSUPPORTED   # block not a multiple of 16
    assert decode(lib, q=FAKE + 4) == PA_ERR_ALIGN
    assert decode(lib, scale=float("inf")) == PA_ERR_SHAPE
    assert decode(lib, scale=float("nan")) == PA_ERR_SHAPE
    # any finite scale, of either sign, passes validation (the next check fails)
    assert decode(lib, scale=-1.0, out=None) == PA_ERR_NULL
    assert decode(lib, scale=-1.0, Hq=16, Hkv=2, out=None) == PA_ERR_NULL
    # two partitions need a workspace
    assert decode(lib, P=16) == PA_ERR_WORKSPACE
    assert decode(lib, S=-1) == PA_ERR_SHAPE
    assert decode(lib, S=0) == PA_OK and lib.pa_last_error() == b""


def test_workspace_and_partition_sizing(lib):
    ws = lib.pa_decode_workspace_bytes
    ps = lib.pa_decode_partition_size
    assert ps(128, 32, 32, 16, 2400, 0) == 1024
    assert ps(64, 32, 8, 16, 993, 0) == 1024      # grouped heads: one partition per sequence
    assert ps(1, 1, 1, 16, 100, 48) == 48
    assert ps(1, 1, 1, 16, 100, 40) == -1
    assert ps(1, 1, 1, 32, 100, 48) == 48        # partitions may start inside a block
    P = ps(16, 32, 32, 32, 4096, 0)
    assert P % 32 == 0
    # more partitions than one round of the vector kernel's resident
    # workgroups (2,048) are split evenly: one more piece per sequence and a
    # piece count per (sequence, KV head)
    assert ws(16, 32, 32, 128, 32, 4096, 512) == 16 * 32 * 9 * 130 * 4 + 16 * 32 * 4
    assert ws(16, 32, 32, 128, 32, 4096, 1024) == 16 * 32 * 4 * 130 * 4   # 2,048: one round
    assert ws(2, 4, 4, 128, 16, 48, 0) == 0              # one partition: no workspace
    assert ws(2, 4, 4, 128, 16, 48, 16) == 2 * 4 * 3 * 130 * 4
    assert ws(1025, 4, 4, 128, 16, 48, 16) == 1025 * 4 * 3 * 130 * 4   # over 1024 sequences


def test_workspace_size_is_exact_or_zero(lib):
    # S * Hq * ceil(L / P) * (D + 2) fp32 values when more than one partition,
    # 0 for one partition, invalid sizes, or a product past 64 bits
    ws = lib.pa_decode_workspace_bytes
    rng = __import__("numpy").random.default_rng(11)
    big = (1 << 31) - 1
    cases = [(1, 1, 1, 128, 16, 4096, 16), (big, big, 1, big, 16, big, 16), (big, 32, 32, 128, 16, big, 16),
             (0, 32, 32, 128, 16, 100, 16), (4, 32, 32, -5, 16, 100, 16), (4, 32, 32, 128, 16, 100, 24)]
    for _ in range(300):
        cases.append((int(rng.integers(0, big)), int(rng.integers(1, 1 << int(rng.integers(1, 31)))), 1,
                      int(rng.integers(1, 1 << int(rng.integers(1, 31)))), 16,
                      int(rng.integers(1, big)), 16 * int(rng.integers(1, 64))))
    for S, Hq, Hkv, D, B, L, P in cases:
        got = ws(S, Hq, Hkv, D, B, L, P)
        if P % 16 or S <= 0 or Hq <= 0 or D <= 0 or L <= 0:
            assert got == 0
            continue
        parts = -(-L // P)
        even = even_split(S, Hq, Hkv, P, parts)
        want = S * Hq * (parts + even) * (D + 2) * 4 + even * S * Hkv * 4 if parts > 1 else 0
        assert got == (want if want < (1 << 64) else 0), (S, Hq, D, L, P, got, want)


def test_workspace_of_the_even_split(lib):
    # one more partial per (sequence, query head) and a piece count per
    # (sequence, KV head) when the work is split evenly
    ws = lib.pa_decode_workspace_bytes
    assert ws(128, 32, 8, 128, 16, 2500, 0) == 128 * 32 * 4 * 130 * 4 + 128 * 8 * 4
    assert ws(128, 64, 8, 128, 16, 2500, 0) == 128 * 64 * 4 * 130 * 4 + 128 * 8 * 4
    # groups of 2 and of 1: 3,072 and 12,288 partitions, more than 2,048
    assert ws(128, 16, 8, 128, 16, 2500, 0) == 128 * 16 * 4 * 130 * 4 + 128 * 8 * 4
    assert ws(128, 32, 32, 128, 16, 2500, 0) == 128 * 32 * 4 * 130 * 4 + 128 * 32 * 4
    # groups of 1 with 1,536 partitions (within one round of the vector kernel):
    # no split, and the default size grows to one partition per sequence
    assert ws(128, 4, 4, 128, 16, 2500, 0) == 0
    assert ws(128, 4, 4, 128, 16, 2500, 1024) == 128 * 4 * 3 * 130 * 4
    assert ws(1025, 32, 8, 128, 16, 2500, 1024) == 1025 * 32 * 3 * 130 * 4  # over 1024 sequences
    assert ws(1025, 32, 8, 128, 16, 2500, 0) == 0   # ... where the default covers each in one
    assert ws(64, 32, 8, 128, 16, 993, 0) == 0                            # one partition
    # split positions past 32 bits: one piece per partition
    assert ws(1024, 32, 8, 128, 16, 1 << 22, 16) == 1024 * 32 * (1 << 18) * 130 * 4
    rng = __import__("numpy").random.default_rng(12)
    for _ in range(300):
        S = int(rng.integers(1, 1200))
        Hkv = int(rng.choice([1, 2, 8]))
        Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
        P = 16 * int(rng.integers(1, 80))
        L = int(rng.integers(1, 200000))
        parts = -(-L // P)
        even = even_split(S, Hq, Hkv, P, parts)
        want = S * Hq * (parts + even) * 130 * 4 + even * S * Hkv * 4 if parts > 1 else 0
        assert ws(S, Hq, Hkv, 128, 16, L, P) == want, (S, Hq, Hkv, L, P)


def test_default_partition_keeps_a_workgroup_per_compute_unit(lib):
    # the library's choice: 1024 tokens, halved while the launch (partitions x
    # sequences x KV heads) would have fewer workgroups than the 256 CUs, down
    # to 64; without an even split and with at least 1,024 such workgroups,
    # doubled while P < L and the doubled size still gives 512; these are the
    # measured best choices for each batch shape
    ps = lib.pa_decode_partition_size
    shapes = [  # S, Hq, Hkv, max_context_len, chosen P
        (1, 32, 32, 1000, 128), (1, 32, 32, 4000, 512), (1, 32, 32, 16000, 1024),
        (4, 32, 32, 2000, 1024), (8, 32, 32, 853, 1024), (8, 32, 8, 2000, 512),
        (16, 32, 32, 4096, 4096), (128, 32, 32, 2400, 1024), (2, 4, 4, 48, 64),
        (32, 32, 32, 4096, 1024), (16, 32, 32, 3000, 4096), (1100, 32, 32, 2000, 2048)]
    for S, Hq, Hkv, L, want in shapes:
        P = ps(S, Hq, Hkv, 16, L, 0)
        assert P == want, (S, Hq, Hkv, L, P)
        wgs = lambda p: S * Hkv * -(-L // p)
        assert P == 64 or wgs(P) >= 256
        assert P >= 1024 or wgs(2 * P) < 256
        if P > 1024:
            assert wgs(P) >= 512 and wgs(P // 2) >= 1024


def test_append_kv_validation(lib):
    v = ctypes.c_void_p
    f = lib.pa_append_kv
    f.argtypes = [v, v, v, v, v, v, v, v, v] + [ctypes.c_int] * 7 + [v]

    def call(slots=None, key=FAKE, val=FAKE, kp=FAKE, vp=FAKE, tables=FAKE, seq=None, pos=None,
             lens=FAKE, T=2, S=2, MB=3, Hkv=2, D=128, B=16, NB=8):
        return f(slots, key, val, kp, vp, tables, seq, pos, lens, T, S, MB, Hkv, D, B, NB, None)

    assert call(T=0) == PA_OK                        # nothing to do
    assert call(T=-1) == PA_ERR_SHAPE
    assert call(MB=0) == PA_ERR_SHAPE
    assert call(D=12) == PA_ERR_UNSUPPORTED
    assert call(T=3, S=2) == PA_ERR_SHAPE            # more tokens than sequences needs seq_ids
    assert call(key=None) == PA_ERR_NULL
    assert call(tables=None) == PA_ERR_NULL
    assert call(lens=None) == PA_ERR_NULL            # neither positions nor lengths
    assert call(kp=FAKE + 8) == PA_ERR_ALIGN
    assert call(slots=FAKE + 4) == PA_ERR_ALIGN


def test_write_copy_slot_validation(lib):
    v = ctypes.c_void_p
    assert lib.pa_write_kv(v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, 4, 2, 128, 16, 8, None) == PA_ERR_NULL
    assert lib.pa_write_kv(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), 4, 2, 12, 16, 8, None) == PA_ERR_UNSUPPORTED
    assert lib.pa_write_kv(v(FAKE + 8), v(FAKE), v(FAKE), v(FAKE), v(FAKE), 4, 2, 128, 16, 8, None) == PA_ERR_ALIGN
    assert lib.pa_write_kv(None, None, None, None, None, 0, 2, 128, 16, 8, None) == PA_OK
    assert lib.pa_copy_blocks(v(FAKE), None, v(FAKE), 3, 2, 128, 16, 8, None) == PA_ERR_NULL
    assert lib.pa_copy_blocks(v(FAKE), v(FAKE), v(FAKE), -1, 2, 128, 16, 8, None) == PA_ERR_SHAPE
    assert lib.pa_copy_blocks(None, None, None, 0, 2, 128, 16, 8, None) == PA_OK
    assert lib.pa_swap_blocks(v(FAKE), v(FAKE), None, v(FAKE), v(FAKE), 2, 2, 128, 16, 8, 8, None) == PA_ERR_NULL
    assert lib.pa_swap_blocks(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), -1, 2, 128, 16, 8, 8, None) == PA_ERR_SHAPE
    assert lib.pa_swap_blocks(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), 2, 2, 12, 16, 8, 8, None) == PA_ERR_UNSUPPORTED
    assert lib.pa_swap_blocks(v(FAKE + 4), v(FAKE), v(FAKE), v(FAKE), v(FAKE), 2, 2, 128, 16, 8, 8, None) == PA_ERR_ALIGN
    assert lib.pa_swap_blocks(None, None, None, None, None, 0, 2, 128, 16, 8, 8, None) == PA_OK
    assert lib.pa_slot_mapping(v(FAKE), v(FAKE), None, None, None, 4, 4, 3, 16, 8, None) == PA_ERR_NULL
    assert lib.pa_slot_mapping(v(FAKE), v(FAKE), None, v(FAKE), None, 5, 4, 3, 16, 8, None) == PA_ERR_SHAPE
    assert lib.pa_slot_mapping(v(FAKE), v(FAKE), None, v(FAKE), None, 4, 4, 3, 0, 8, None) == PA_ERR_SHAPE


def test_package_refuses_to_import_without_the_library(tmp_path):
    # a copy of the package without libpa.so must fail loudly, never fall back
    import shutil
    import subprocess
    import sys
    dst = tmp_path / "paged_kv_cache_151_amd"
    shutil.copytree(os.path.join(ROOT, "paged_kv_cache_151_amd"), dst,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    r = subprocess.run([sys.executable, "-c", "import paged_kv_cache_151_amd"], cwd=tmp_path,
                       capture_output=True, text=True)
    assert r.returncode != 0 and "libpa.so is missing" in r.stderr


def prefill(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, t=FAKE, l=FAKE, qs=FAKE, S=2, T=40, Hq=4, Hkv=4,
             D=128, B=16, NB=16, MB=3, maxq=32, scale=0.1)
    a.update(kw)
    v = ctypes.c_void_p
    return lib.pa_prefill(v(a["out"]), v(a["q"]), v(a["k"]), v(a["v"]), v(a["t"]), v(a["l"]),
                          v(a["qs"]), a["S"], a["T"], a["Hq"], a["Hkv"], a["D"], a["B"], a["NB"],
                          a["MB"], a["maxq"], F(a["scale"]), None)


def test_prefill_host_validation(lib):
    assert prefill(lib, qs=None) == PA_ERR_NULL
    assert prefill(lib, Hq=6, Hkv=4) == PA_ERR_SHAPE
    assert prefill(lib, D=64) == PA_ERR_UNSUPPORTED
    assert prefill(lib, B=24, MB=2) == PA_ERR_UNSUPPORTED
    assert prefill(lib, B=8, MB=6, out=None) == PA_ERR_NULL     # B = 8 passes validation
    assert prefill(lib, Hq=12, Hkv=4) == PA_ERR_UNSUPPORTED    # group of 3
    assert prefill(lib, maxq=41) == PA_ERR_SHAPE               # more rows than T
    assert prefill(lib, maxq=-1) == PA_ERR_SHAPE
    assert prefill(lib, T=-1) == PA_ERR_SHAPE
    assert prefill(lib, out=FAKE + 2) == PA_ERR_ALIGN
    assert prefill(lib, qs=FAKE + 2) == PA_ERR_ALIGN
    assert prefill(lib, scale=float("nan")) == PA_ERR_SHAPE
    # any finite scale, of either sign, passes validation (the next check fails)
    assert prefill(lib, scale=-0.5, out=None) == PA_ERR_NULL
    assert prefill(lib, S=0) == PA_OK
    assert prefill(lib, maxq=0, out=None) == PA_OK



def test_launch_size_limits(lib):
    """Shapes whose launch would not fit a dispatch packet (a 32-bit count of
    work-items) are refused as shape errors before any pointer is looked at;
    the largest shapes that fit get as far as the null-pointer check."""
    v = ctypes.c_void_p
    # decode: one workgroup of 2 waves per (sequence, KV head) at group size 1
    assert decode(lib, out=None, S=2**23 - 1, Hq=4, Hkv=4, MB=3, maxL=48) == PA_ERR_NULL
    assert decode(lib, out=None, S=2**23, Hq=4, Hkv=4, MB=3, maxL=48) == PA_ERR_SHAPE
    # prefill, group size 1: 64 rows and 256 threads per workgroup, grid padded to 8
    assert prefill(lib, out=None, S=2**20, T=64, Hq=15, Hkv=15, maxq=64) == PA_ERR_NULL
    assert prefill(lib, out=None, S=2**20, T=64, Hq=16, Hkv=16, maxq=64) == PA_ERR_SHAPE
    # write_kv: one work-item per 16-byte chunk, T * Hkv * D / 8 of them
    assert lib.pa_write_kv(None, None, None, None, None, 2**26 - 4, 4, 128, 16, 8, None) == PA_ERR_NULL
    assert lib.pa_write_kv(None, None, None, None, None, 2**26 - 3, 4, 128, 16, 8, None) == PA_ERR_SHAPE
    # copy and swap: one block of Hkv * B * D fp16 must fit one launch
    assert lib.pa_copy_blocks(None, None, None, 1, 2**14, 2**14, 128, 8, None) == PA_ERR_NULL
    assert lib.pa_copy_blocks(None, None, None, 0, 2**16, 2**16, 128, 8, None) == PA_ERR_SHAPE
    assert lib.pa_swap_blocks(None, None, None, None, None, 0, 2**16, 2**16, 128, 8, 8, None) == PA_ERR_SHAPE

def test_stream_read_host_validation(lib):
    v = ctypes.c_void_p
    lib.pa_stream_read.argtypes = [v, ctypes.c_size_t, v, ctypes.c_int, v]
    assert lib.pa_stream_read(v(FAKE), 4096, None, 64, None) == PA_ERR_NULL
    assert lib.pa_stream_read(v(FAKE), 4090, v(FAKE), 64, None) == PA_ERR_SHAPE
    assert lib.pa_stream_read(v(FAKE), 4096, v(FAKE), 0, None) == PA_ERR_SHAPE
    assert lib.pa_stream_read(v(FAKE + 8), 4096, v(FAKE), 64, None) == PA_ERR_ALIGN
    assert lib.pa_stream_read(None, 0, None, 64, None) == PA_OK


def test_binding_refuses_tensors_it_would_misread():
    # checked in the binding before any library call, so this runs without a GPU
    import torch
    import paged_kv_cache_151_amd as pa
    key = torch.zeros(4, 2, 128, dtype=torch.float16)
    pool = torch.zeros(8, 2, 16, 128, dtype=torch.float16)
    slots = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError, match="device tensor"):
        pa.pa_write_kv(key, key, pool, pool, slots)
    with pytest.raises(TypeError, match="float16"):
        pa.pa_write_kv(key.float(), key, pool, pool, slots)
    strided = torch.zeros(4, 4, 128, dtype=torch.float16)[:, ::2]   # [4, 2, 128], not contiguous
    with pytest.raises(ValueError, match="contiguous"):
        pa.pa_write_kv(strided, strided, pool, pool, slots)
    with pytest.raises(ValueError, match="differ"):
        pa.pa_write_kv(key, key[:3], pool, pool, slots)
    with pytest.raises(TypeError, match="int32"):   # an int64 block mapping would be misread
        pa._arg(torch.zeros(2, 2, dtype=torch.int64), "block_mapping", torch.int32)


def test_binding_refuses_arrays_shorter_than_the_sizes_it_passes():
    # the kernels index these arrays by sequence, token or pair: a short one
    # would be read past its end, so the binding refuses it (CPU tensors: the
    # shape checks come before any device check or library call)
    import torch
    import paged_kv_cache_151_amd as pa
    f16, i32, i64 = torch.float16, torch.int32, torch.int64
    q = torch.zeros(3, 4, 128, dtype=f16)
    pool = torch.zeros(8, 4, 16, 128, dtype=f16)
    with pytest.raises(ValueError, match="block_tables needs 3 rows"):
        pa.pa_decode(q, pool, pool, torch.zeros(2, 4, dtype=i32), torch.zeros(3, dtype=i32), 48, 0.1)
    with pytest.raises(ValueError, match="context_lens needs 3 rows"):
        pa.pa_decode(q, pool, pool, torch.zeros(3, 4, dtype=i32), torch.zeros(2, dtype=i32), 48, 0.1)
    key = torch.zeros(5, 4, 128, dtype=f16)
    with pytest.raises(ValueError, match="slot_mapping needs 5 rows"):
        pa.pa_write_kv(key, key, pool, pool, torch.zeros(4, dtype=i64))
    with pytest.raises(ValueError, match="does not fit pool blocks"):
        pa.pa_write_kv(key[:, :2].contiguous(), key[:, :2].contiguous(), pool, pool,
                       torch.zeros(5, dtype=i64))
    with pytest.raises(ValueError, match=r"\[n, 2\]"):
        pa.pa_copy_blocks(pool, pool, torch.zeros(6, dtype=i32))
    with pytest.raises(ValueError, match=r"\[n, 2\]"):
        pa.pa_swap_blocks(pool, pool, pool, pool, torch.zeros(3, 3, dtype=i32))
    tables = torch.zeros(2, 4, dtype=i32)
    with pytest.raises(ValueError, match="seq_ids needs 5 rows"):
        pa.pa_slot_mapping(tables, 16, 8, seq_ids=torch.zeros(4, dtype=i32),
                           positions=torch.zeros(5, dtype=i32))
    with pytest.raises(ValueError, match="context_lens needs 2 rows"):
        pa.pa_slot_mapping(tables, 16, 8, context_lens=torch.zeros(1, dtype=i32))
    # index vectors with extra dimensions would be read as flat arrays
    with pytest.raises(ValueError, match="context_lens must have 1 dimension"):
        pa.pa_decode(q, pool, pool, torch.zeros(3, 4, dtype=i32), torch.zeros(3, 2, dtype=i32), 48, 0.1)
    with pytest.raises(ValueError, match="seq_ids must have 1 dimension"):
        pa.pa_slot_mapping(tables, 16, 8, seq_ids=torch.zeros(5, 1, dtype=i32),
                           positions=torch.zeros(5, dtype=i32))
    with pytest.raises(ValueError, match="k_pool must have 4 dimensions"):
        pa.pa_copy_blocks(pool[0], pool[0], torch.zeros(2, 2, dtype=i32))
    with pytest.raises(ValueError, match="key must have 3 dimensions"):
        pa.pa_write_kv(key[0], key[0], pool, pool, torch.zeros(5, dtype=i64))
    with pytest.raises(ValueError, match="src_k_pool must have 4 dimensions"):
        pa.pa_swap_blocks(pool, pool, pool[0], pool[0], torch.zeros(2, 2, dtype=i32))
    buf = torch.zeros(1024, dtype=torch.uint8)
    with pytest.raises(ValueError, match="outside the buffer"):
        pa.pa_stream_read(buf, torch.zeros(1, dtype=i32), nbytes=2048)
    with pytest.raises(ValueError, match="sink needs 4 bytes"):
        pa.pa_stream_read(buf, torch.zeros(2, dtype=torch.uint8))


def test_binding_refuses_pools_that_do_not_fit_the_query():
    # a pool whose rows are shorter than the query's head dimension would be
    # read past its end by the kernels; a 3-D pool or query is misread
    import torch
    import paged_kv_cache_151_amd as pa
    f16, i32 = torch.float16, torch.int32
    q = torch.zeros(3, 4, 128, dtype=f16)
    short = torch.zeros(8, 4, 16, 64, dtype=f16)
    pool = torch.zeros(8, 4, 16, 128, dtype=f16)
    tables, lens = torch.zeros(3, 4, dtype=i32), torch.zeros(3, dtype=i32)
    with pytest.raises(ValueError, match="head dimension 128"):
        pa.pa_decode(q, short, short, tables, lens, 48, 0.1)
    with pytest.raises(ValueError, match="differ"):
        pa.pa_decode(q, pool, short, tables, lens, 48, 0.1)
    with pytest.raises(ValueError, match="k_pool must have 4 dimensions"):
        pa.pa_decode(q, pool[0], pool[0], tables, lens, 48, 0.1)
    with pytest.raises(ValueError, match="query must have 3 dimensions"):
        pa.pa_decode(q[0], pool, pool, tables, lens, 48, 0.1)
    qs = torch.zeros(4, dtype=i32)
    with pytest.raises(ValueError, match="head dimension 128"):
        pa.pa_prefill(q, short, short, tables, lens, qs, 1, 0.1)
    with pytest.raises(ValueError, match="block_tables must have 2 dimensions"):
        pa.pa_prefill(q, pool, pool, tables[0], lens, qs, 1, 0.1)
    with pytest.raises(ValueError, match="query_start S"):
        pa.pa_prefill(q, pool, pool, tables, lens, qs[:3], 1, 0.1)


def test_static_decode_refuses_partials_beyond_its_scratch(lib):
    # the size check comes before the library touches the device
    lib.pa_decode_static_scratch_bytes.restype = ctypes.c_size_t
    cap = lib.pa_decode_static_scratch_bytes()
    assert cap == 32 << 20
    v = ctypes.c_void_p
    S, H, MB, maxL, P = 128, 32, 2000, 32000, 16     # 2000 partitions of partials per head
    need = lib.pa_decode_workspace_bytes(S, H, H, 128, 16, maxL, P)
    assert need > cap
    st = lib.pa_decode_static(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), S, H, H, 128,
                              16, 4096, MB, maxL, F(0.1), P, None)
    assert st == PA_ERR_WORKSPACE
    assert b"static scratch" in lib.pa_last_error()
    assert lib.pa_decode_static(None, v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), 2, 4, 4, 128,
                                16, 16, 3, 48, F(0.1), 0, None) == PA_ERR_NULL


def test_error_details_are_per_thread(lib):
    # the library's only state is a thread-local error string: threads whose
    # calls fail at the same time each read back their own detail (ctypes
    # releases the interpreter lock around foreign calls, so they interleave)
    import threading
    v = ctypes.c_void_p
    bad = []

    def worker(k):
        for i in range(3000):
            T = -(1000 * k + i % 997) - 1
            st = lib.pa_write_kv(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), T, 2, 128, 16, 8, None)
            msg = lib.pa_last_error().decode()
            if st != PA_ERR_SHAPE or f"T={T} " not in msg:
                bad.append((k, i, st, msg))
                return

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad[:3]
