"""Parity of pa_decode and pa_prefill against the fp64 oracle on peaked score
distributions: late keys that dominate every earlier one, scores that rise
along the walk, a large scale and negative scales.

On the flat N(0, 1) workloads a running maximum almost never moves after the
first keys; here it must, repeatedly, which is what the matrix-core kernels'
lazy rescaling (groups of 4 and 8 query heads in decode, every group size in
prefill) exists for. Each case first checks on the host, from the fp64 scores,
that its walks really raise a running maximum by more than 2^8 after the first
unit (decode) or chunk (prefill), so that the branch is taken; then the GPU
output is compared element by element with the oracle at the usual tolerance.
The closed form of a single dominant key (output equal to that token's value
row, [L] "Paged Attention: OS-Inspired Memory Management for KV Caches", "How
PagedAttention works", step 4: attention through the table is attention over
the contiguous tokens) is checked directly as well.
"""
import numpy as np
import pytest

import oracle
import peaked_inputs as PK
import workloads as W
from gpu_util import assert_attention_close, dev, host, pa_module, say
from host_validate import decode_inputs, prefill_inputs

pytestmark = pytest.mark.gpu

SCALE = 1.0 / np.sqrt(W.HEAD_DIM)
DECODE_LENS = [1, 2, 17, 300, 700, 1023, 1500, 2100]
DECODE_FAMILIES = ["dominant", "ramp", "scale_one", "negative_scale", "negative_scale_one"]


@pytest.fixture(scope="module")
def pa():
    return pa_module()


def decode_case(family, G, B, seed):
    c = W.make_case(f"peaked_{family}_G{G}_B{B}", seed, DECODE_LENS, Hq=2 * G, Hkv=2, B=B)
    rng = np.random.default_rng(seed + 1)
    if family == "dominant":
        PK.decode_dominant_keys(c, rng)
    elif family == "ramp":
        PK.decode_ramp(c)
    elif family == "scale_one":
        c.scale = 1.0
    elif family == "negative_scale":
        c.scale = -SCALE
        PK.decode_dominant_keys(c, rng)
    elif family == "negative_scale_one":
        c.scale = -1.0
    return c


def decode_gpu(pa, c, P):
    tables, lens = dev(c.block_tables), dev(c.context_lens)
    kp, vp = dev(c.k_pool), dev(c.v_pool)
    slots = pa.pa_slot_mapping(tables, c.B, c.NB, context_lens=lens)
    pa.pa_write_kv(dev(c.key_new), dev(c.value_new), kp, vp, slots)
    out = pa.pa_decode(dev(c.query), kp, vp, tables, lens, c.max_context_len, c.scale,
                       partition_size=P)
    return host(out)


def decode_oracle(c):
    slots = oracle.decode_slots(c.block_tables, c.context_lens, c.B, c.NB)
    kp, vp = oracle.write_kv(c.k_pool, c.v_pool, c.key_new, c.value_new, slots)
    return oracle.decode(c.query, kp, vp, c.block_tables, c.context_lens, c.scale)


@pytest.mark.parametrize("B", [8, 16, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("family", DECODE_FAMILIES)
def test_decode_peaked_scores(pa, family, G, B):
    c = decode_case(family, G, B, 9000 + 100 * DECODE_FAMILIES.index(family) + 10 * G + B)
    decode_inputs(c.block_tables, c.context_lens, c.B, c.NB, c.max_context_len)
    ref = decode_oracle(c)
    for P in (0, 64, 1024):
        Pe = pa.pa_decode_partition_size(c.S, c.Hq, c.Hkv, c.B, c.max_context_len, P)
        rises, walks = PK.decode_rescale_count(c, Pe)
        # 1024-token partitions give each of 4 waves up to 16 units to walk (with
        # 64-token ones each wave has a single unit: nothing to raise)
        if P == 1024:
            assert rises > 0, f"{c.name}: no walk raises its maximum at P={Pe}"
        say(c.name, f"scale={c.scale:.4g} P={P} (effective {Pe}): {rises} of {walks} "
                    f"multi-unit walks raise their maximum by more than 2^8")
        assert_attention_close(decode_gpu(pa, c, P), ref, f"{c.name} P={P}")


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_single_dominant_key_gives_its_value_row(pa, G):
    """The closed form: one key per (sequence, KV head) scores at least 24 log2
    units above every other key for every head of its group, so the output is
    that token's value row (the other tokens' total weight is below 2^-12)."""
    c = W.make_case(f"dominant_one_G{G}", 9500 + G, DECODE_LENS[1:], Hq=2 * G, Hkv=2, B=16)
    where = PK.decode_dominant_keys(c, np.random.default_rng(9600 + G), n_keys=1, first_gap=80.0)
    want = np.empty((c.S, c.Hq, c.D))
    for s in range(c.S):
        L = int(c.context_lens[s])
        V = oracle.gather(c.v_pool, c.block_tables[s], L, c.B).astype(np.float64)
        V[:, L - 1] = c.value_new[s]
        for h in range(c.Hq):
            g = h // G
            t = int(where[(s, g)][0])
            sc = PK.decode_scores_log2(c, s, h)
            gap = sc[t] - np.delete(sc, t).max()
            assert gap >= 24, f"seq {s} head {h}: dominant key only {gap:.1f} log2 units ahead"
            want[s, h] = V[g, t]
    say(c.name, "closed form")
    for P in (0, 64, 1024):
        assert_attention_close(decode_gpu(pa, c, P), want, f"{c.name} P={P}")


PREFILL_NEW = [1, 15, 70, 130, 300, 64]
PREFILL_CACHED = [0, 40, 0, 500, 20, 3]


def prefill_case(family, G, B, seed):
    c = W.make_prefill_case(f"peaked_prefill_{family}_G{G}_B{B}", seed, PREFILL_NEW,
                            PREFILL_CACHED, Hq=2 * G, Hkv=2, B=B)
    rng = np.random.default_rng(seed + 1)
    if family == "scale_one":
        c.scale = 1.0
        return c
    if family == "negative_scale_one":
        c.scale = -1.0
        return c
    if family == "negative_scale":
        c.scale = -SCALE
    dirs = PK.prefill_shared_direction(c, rng)
    if family == "ramp":
        PK.prefill_ramp(c, dirs)
    else:
        PK.prefill_dominant_keys(c, rng, dirs)
    return c


PREFILL_FAMILIES = ["dominant", "ramp", "scale_one", "negative_scale", "negative_scale_one"]


@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("family", PREFILL_FAMILIES)
def test_prefill_peaked_scores(pa, family, G):
    for B in (16,) if family != "dominant" else (8, 16, 32):
        c = prefill_case(family, G, B, 9700 + 100 * PREFILL_FAMILIES.index(family) + 10 * G + B)
        prefill_inputs(c.block_tables, c.context_lens, c.query_start, c.T, c.B, c.NB,
                       c.max_query_len)
        hits, rows = PK.prefill_rescale_rows(c)
        assert hits > 0, f"{c.name}: no row raises its maximum after the first chunk"
        say(c.name, f"scale={c.scale:.4g}: {hits} of {rows} (row, head) pairs raise their "
                    f"maximum by more than 2^8 after the first 32 keys")
        got = host(pa.pa_prefill(dev(c.query), dev(c.k_pool), dev(c.v_pool), dev(c.block_tables),
                                 dev(c.context_lens), dev(c.query_start), c.max_query_len,
                                 c.scale))
        ref = oracle.prefill(c.query, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                             c.query_start, c.scale)
        assert_attention_close(got, ref, c.name)


# ---------------------------------------------------------------------------
# The remaining closed forms of decode, on the GPU for every group size (both
# kernels): the pages fix the result as attention over the contiguous tokens
# ([L] "How PagedAttention works", step 4; "Key takeaways": paging is exact),
# and for these inputs that attention has a value that needs no oracle.
# ---------------------------------------------------------------------------

def _closed_form_case(name, seed, G, lens, B=16):
    return W.make_case(name, seed, lens, Hq=2 * G, Hkv=2, B=B)


def _values_in_order(c, s):
    """Value rows of sequence s in logical order, the new token included: [Hkv, L, D]."""
    L = int(c.context_lens[s])
    V = oracle.gather(c.v_pool, c.block_tables[s], L, c.B).astype(np.float64)
    V[:, L - 1] = c.value_new[s]
    return V


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_single_token_gives_its_value_row_bit_exact(pa, G):
    """L = 1: the one weight is 1, so the output is V_0 exactly (fp16 in, fp16 out)."""
    c = _closed_form_case(f"one_token_G{G}", 9800 + G, G, [1, 1, 1, 1])
    say(c.name)
    for P in (0, 16):
        got = decode_gpu(pa, c, P)
        want = np.repeat(c.value_new, G, axis=1)          # query head h reads KV head h // G
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), f"{c.name} P={P}"


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_zero_query_or_equal_keys_give_the_mean_of_values(pa, G):
    """Every score equal (a zero query; or one key repeated at every position):
    the weights are uniform and the output is the mean of the value rows."""
    lens = [3, 17, 100, 1030, 2049]
    for how in ("zero query", "equal keys"):
        c = _closed_form_case(f"uniform_{how.replace(' ', '_')}_G{G}", 9810 + G, G, lens)
        if how == "zero query":
            c.query[:] = 0
        else:
            rng = np.random.default_rng(9820 + G)
            for s in range(c.S):
                L = int(c.context_lens[s])
                key = W.f16_normal(rng, (c.Hkv, c.D))
                c.key_new[s] = key
                for t in range(L - 1):
                    for g in range(c.Hkv):
                        PK._set_key(c.k_pool, c.block_tables[s], t, c.B, g, key[g])
        want = np.stack([np.repeat(_values_in_order(c, s).mean(axis=1), G, axis=0)
                         for s in range(c.S)])
        say(c.name, how)
        for P in (0, 64, 1024):
            assert_attention_close(decode_gpu(pa, c, P), want, f"{c.name} P={P}")


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_constant_values_give_that_constant(pa, G):
    """Every value row equal to one vector: whatever the weights, the output is
    that vector (to the fp16 rounding of the weights on the matrix cores)."""
    c = _closed_form_case(f"constant_values_G{G}", 9830 + G, G, [2, 40, 513, 1500])
    PK.decode_dominant_keys(c, np.random.default_rng(9840 + G))    # peaked weights too
    const = W.f16_normal(np.random.default_rng(9850 + G), (c.Hkv, c.D))
    c.v_pool[:] = const[None, :, None, :]
    c.value_new[:] = const[None]
    want = np.broadcast_to(np.repeat(const, G, axis=0)[None].astype(np.float64), (c.S, c.Hq, c.D))
    say(c.name)
    for P in (0, 64, 1024):
        assert_attention_close(decode_gpu(pa, c, P), want, f"{c.name} P={P}")
