"""The bounds-checked debug build (libpa_debug.so) on the GPU.

Every global-memory access of its kernels is compared with the extent of its
buffer first; an access that would leave it is suppressed and counted. Two
kinds of cases run through it here, each checked on the host to be counted
zero times at every site:
  * valid input across the paths (vector and matrix-core decode, the even
    split, every block-size specialisation, prefill, the cache calls), where
    the outputs also match the oracle;
  * input that breaks the caller's contract in the ways the header says the
    kernels contain: lengths past the table, table entries outside the pool,
    negative lengths, slots and copy pairs outside the pools, query ranges
    outside the packed rows. The results are unspecified; the zero counts show
    that the clamps keep every access inside its buffer.
The module switches the binding to the debug library and back."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_attention_close, dev, host, pa_module, say, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    m = pa_module()
    before = m.use_library(m.DEBUG_LIB_PATH)
    assert m.pa_debug_bounds_violations() is not None, "debug library not in use"
    yield m
    m.use_library(before)


def test_the_counting_path_reports_what_is_counted(pa):
    # every source file's counters reach the host: one refusal per site each
    pa.pa_debug_bounds_violations()
    files = pa.pa_debug_bounds_selftest()
    assert files == 4
    v = pa.pa_debug_bounds_violations()
    assert set(v) == {"length", "table", "query", "pool", "out", "partial", "slot", "pair"}
    assert all(n == files for n in v.values()), v
    assert not any(pa.pa_debug_bounds_violations().values())   # read and cleared


def no_violations(pa, what):
    v = pa.pa_debug_bounds_violations()
    assert v is not None and not any(v.values()), f"{what}: refused accesses {v}"


def decode(pa, c, kp=None, vp=None, tables=None, lens=None, max_len=None, P=0):
    return host(pa.pa_decode(dev(c.query), dev(c.k_pool if kp is None else kp),
                             dev(c.v_pool if vp is None else vp),
                             dev(c.block_tables if tables is None else tables),
                             dev(c.context_lens if lens is None else lens),
                             c.max_context_len if max_len is None else max_len, c.scale,
                             partition_size=P))


@pytest.mark.parametrize("B", [8, 16, 32, 48])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_valid_input_is_never_refused(pa, G, B):
    pa.pa_debug_bounds_violations()   # start from zero
    lens = [0, 1, 15, 16, 17, 100, 700, 1025]
    c = W.make_case(f"dbg_G{G}_B{B}", 7000 + 10 * G + B, lens, Hq=2 * G, Hkv=2, B=B)
    ref = oracle.decode(c.query, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale)
    for P in (0, 64):
        say(c.name, f"debug build, P={P}")
        assert_attention_close(decode(pa, c, P=P), ref, c.name)
        no_violations(pa, f"{c.name} P={P}")


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (64, 64)])
def test_even_split_and_static_scratch_are_never_refused(pa, Hq, Hkv):
    # groups of 4 (matrix cores) and of 1 (vector kernel; 64 KV heads give it
    # enough partitions to take the split)
    pa.pa_debug_bounds_violations()
    c = W.make_case(f"dbg_even_{Hq}_{Hkv}", 7100, [0, 900, 33, 1500, 1, 260, 0, 640], Hq=Hq, Hkv=Hkv,
                    B=16)
    ref = oracle.decode(c.query, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale)
    say(c.name, "debug build, even split and static scratch")
    assert_attention_close(decode(pa, c, P=64), ref, c.name)
    out = pa.pa_decode_static(dev(c.query), dev(c.k_pool), dev(c.v_pool), dev(c.block_tables),
                              dev(c.context_lens), c.max_context_len, c.scale, partition_size=64)
    assert_attention_close(host(out), ref, c.name + " static")
    no_violations(pa, c.name)


@pytest.mark.parametrize("B", [8, 16])
@pytest.mark.parametrize("G", [1, 4])
def test_prefill_valid_input_is_never_refused(pa, G, B):
    pa.pa_debug_bounds_violations()
    c = W.make_prefill_case(f"dbg_prefill_G{G}_B{B}", 7200 + G + B, [1, 17, 65, 130, 33],
                            [0, 5, 100, 31, 0], Hq=2 * G, Hkv=2, B=B)
    say(c.name, "debug build")
    got = host(pa.pa_prefill(dev(c.query), dev(c.k_pool), dev(c.v_pool), dev(c.block_tables),
                             dev(c.context_lens), dev(c.query_start), c.max_query_len, c.scale))
    ref = oracle.prefill(c.query, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                         c.query_start, c.scale)
    assert_attention_close(got, ref, c.name)
    no_violations(pa, c.name)


def test_cache_calls_valid_input_is_never_refused(pa):
    pa.pa_debug_bounds_violations()
    c = W.make_case("dbg_cache", 7300, [40, 17, 64], Hq=4, Hkv=4, B=16)
    say(c.name, "debug build: slots, store, copy")
    kp, vp = dev(c.k_pool), dev(c.v_pool)
    tables, lens = dev(c.block_tables), dev(c.context_lens)
    slots = pa.pa_slot_mapping(tables, c.B, c.NB, context_lens=lens)
    pa.pa_write_kv(dev(c.key_new), dev(c.value_new), kp, vp, slots)
    ref_slots = oracle.decode_slots(c.block_tables, c.context_lens, c.B, c.NB)
    rk, rv = oracle.write_kv(c.k_pool, c.v_pool, c.key_new, c.value_new, ref_slots)
    assert np.array_equal(host(slots), ref_slots)
    used = set(c.block_tables[c.block_tables >= 0].tolist())
    free = [b for b in range(c.NB) if b not in used]
    # distinct destinations that no pair reads, so the copies do not depend on order
    pairs = np.array([[c.block_tables[0, 0], free[0]], [c.block_tables[1, 1], free[1]]], np.int32)
    pa.pa_copy_blocks(kp, vp, dev(pairs))
    rk, rv = oracle.copy_blocks(rk, rv, pairs)
    assert np.array_equal(u16(host(kp)), u16(rk)) and np.array_equal(u16(host(vp)), u16(rv))
    no_violations(pa, c.name)


@pytest.mark.parametrize("G", [1, 4])
def test_decode_contract_breaches_stay_inside_the_buffers(pa, G):
    pa.pa_debug_bounds_violations()
    c = W.make_case(f"dbg_breach_G{G}", 7400 + G, [100, 300, 64, 500], Hq=4 * G, Hkv=4, B=16)
    MB = c.block_tables.shape[1]
    tables = c.block_tables.copy()
    tables[0, 1] = c.NB + 5          # entries outside the pool, inside the used range
    tables[1, 0] = -3
    tables[3, 2] = np.iinfo(np.int32).max
    lens = c.context_lens.copy()
    lens[2] = MB * c.B + 50          # past the table
    lens[1] = -7                     # negative
    say(c.name, "debug build, contract breaches")
    for P in (0, 16):
        out = decode(pa, c, tables=tables, lens=lens, max_len=MB * c.B, P=P)
        assert out.shape == c.query.shape
        no_violations(pa, f"{c.name} P={P}")


def test_prefill_contract_breaches_stay_inside_the_buffers(pa):
    pa.pa_debug_bounds_violations()
    c = W.make_prefill_case("dbg_prefill_breach", 7500, [20, 40, 9], [10, 0, 70], Hq=8, Hkv=2, B=16)
    tables = c.block_tables.copy()
    tables[0, 0] = c.NB + 1
    tables[2, 1] = -1
    lens = c.context_lens.copy()
    lens[0] = c.block_tables.shape[1] * c.B + 33   # past the table
    qs = c.query_start.copy()
    qs[2] = qs[3] + 5                # a range past the packed rows: untouched
    say(c.name, "debug build, contract breaches")
    pa.pa_prefill(dev(c.query), dev(c.k_pool), dev(c.v_pool), dev(tables), dev(lens), dev(qs),
                  c.max_query_len, c.scale)
    no_violations(pa, c.name)


def test_cache_call_breaches_stay_inside_the_buffers(pa):
    pa.pa_debug_bounds_violations()
    c = W.make_case("dbg_cache_breach", 7600, [40, 17], Hq=2, Hkv=2, B=16)
    kp, vp = dev(c.k_pool), dev(c.v_pool)
    say(c.name, "debug build, slots and pairs outside the pools")
    slots = np.array([-1, c.NB * c.B], np.int64)
    pa.pa_write_kv(dev(c.key_new), dev(c.value_new), kp, vp, dev(slots))
    pairs = np.array([[c.NB, 0], [0, -1], [-5, c.NB + 2]], np.int32)
    pa.pa_copy_blocks(kp, vp, dev(pairs))
    tables = c.block_tables.copy()
    tables[0, 2] = c.NB + 9
    tables[1, 1] = -4
    pa.pa_slot_mapping(dev(tables), c.B, c.NB, context_lens=dev(c.context_lens))
    # the last token of each sequence lands in those entries: both skipped
    pa.pa_append_kv(dev(c.key_new), dev(c.value_new), kp, vp, dev(tables),
                    context_lens=dev(c.context_lens))
    assert np.array_equal(u16(host(kp)), u16(c.k_pool))   # nothing was written
    no_violations(pa, c.name)
