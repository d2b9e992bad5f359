"""Python binding of libpa.so: paged KV-cache decode on MI355X (gfx950).

Argument marshalling only. Every function passes device pointers of torch
tensors, their sizes and torch's current HIP stream to the C entry point of the
same name (declared in include/pa.h); all work runs in the library's kernels.
Output tensors and the decode workspace are allocated here with torch when the
caller does not pass them. There is no fallback: importing this package fails
when libpa.so has not been built, and every call raises PaError on a non-OK
status.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")
# the same library with every kernel's global-memory accesses bounds-checked
# (python paged_kv_cache_151_amd/build.py --debug); see use_library
DEBUG_LIB_PATH = os.path.join(_PKG, "libpa_debug.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python paged_kv_cache_151_amd/build.py`")

_p = ctypes.c_void_p
_i = ctypes.c_int


def _declare(_lib):
    """Sets the argument and result types of every entry point of `_lib`."""
    _lib.pa_debug_bounds_violations.restype = _i
    _lib.pa_debug_bounds_violations.argtypes = [_p, _i]
    _lib.pa_debug_bounds_site.restype = ctypes.c_char_p
    _lib.pa_debug_bounds_site.argtypes = [_i]
    _lib.pa_debug_bounds_selftest.restype = _i
    _lib.pa_debug_bounds_selftest.argtypes = []
    _lib.pa_status_str.restype = ctypes.c_char_p
    _lib.pa_status_str.argtypes = [_i]
    _lib.pa_last_error.restype = ctypes.c_char_p
    _lib.pa_last_error.argtypes = []
    _lib.pa_version.restype = _i
    _lib.pa_slot_mapping.restype = _i
    _lib.pa_slot_mapping.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p]
    _lib.pa_write_kv.restype = _i
    _lib.pa_write_kv.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p]
    _lib.pa_append_kv.restype = _i
    _lib.pa_append_kv.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i,
                                  _p]
    _lib.pa_copy_blocks.restype = _i
    _lib.pa_copy_blocks.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _p]
    _lib.pa_swap_blocks.restype = _i
    _lib.pa_swap_blocks.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p]
    _lib.pa_decode_partition_size.restype = _i
    _lib.pa_decode_partition_size.argtypes = [_i, _i, _i, _i, _i, _i]
    _lib.pa_decode_workspace_bytes.restype = ctypes.c_size_t
    _lib.pa_decode_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i]
    _lib.pa_decode.restype = _i
    _lib.pa_decode.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i,
                               ctypes.c_float, _i, _p, ctypes.c_size_t, _p]
    _lib.pa_decode_static.restype = _i
    _lib.pa_decode_static.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i,
                                      ctypes.c_float, _i, _p]
    _lib.pa_decode_static_scratch_bytes.restype = ctypes.c_size_t
    _lib.pa_decode_static_scratch_bytes.argtypes = []

    _lib.pa_prefill.restype = _i
    _lib.pa_prefill.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                                ctypes.c_float, _p]
    _lib.pa_stream_read.restype = _i
    _lib.pa_stream_read.argtypes = [_p, ctypes.c_size_t, _p, _i, _p]
    _lib.pa_bm_create.restype = _i
    _lib.pa_bm_create.argtypes = [_i, _i, _i, ctypes.POINTER(_p)]
    _lib.pa_bm_destroy.restype = None
    _lib.pa_bm_destroy.argtypes = [_p]
    _lib.pa_bm_add_sequence.restype = _i
    _lib.pa_bm_add_sequence.argtypes = [_p, ctypes.POINTER(_i)]
    _lib.pa_bm_fork.restype = _i
    _lib.pa_bm_fork.argtypes = [_p, _i, ctypes.POINTER(_i)]
    _lib.pa_bm_append_tokens.restype = _i
    _lib.pa_bm_append_tokens.argtypes = [_p, _p, _i, _p, _p, _i, ctypes.POINTER(_i), ctypes.POINTER(_i)]
    _lib.pa_bm_release.restype = _i
    _lib.pa_bm_release.argtypes = [_p, _i, ctypes.POINTER(_i)]
    _lib.pa_bm_get_table.restype = _i
    _lib.pa_bm_get_table.argtypes = [_p, _i, _p, _i, ctypes.POINTER(_i), ctypes.POINTER(ctypes.c_int64)]
    _lib.pa_bm_export.restype = _i
    _lib.pa_bm_export.argtypes = [_p, _p, _i, _p, _i, _p]
    _lib.pa_bm_num_free.restype = _i
    _lib.pa_bm_num_free.argtypes = [_p]
    _lib.pa_bm_refcount.restype = _i
    _lib.pa_bm_refcount.argtypes = [_p, _i]
    return _lib


_lib = _declare(ctypes.CDLL(LIB_PATH))


def use_library(path: str = LIB_PATH) -> str:
    """Routes every following call to the library at `path` (for example
    DEBUG_LIB_PATH, the bounds-checked build); returns the path in use before.
    Tensors, streams and results are unaffected: both libraries take the same
    arguments."""
    global _lib, _lib_path
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with paged_kv_cache_151_amd/build.py")
    before = _lib_path
    _lib = _declare(ctypes.CDLL(path))
    _lib_path = path
    return before


_lib_path = LIB_PATH

PA_OK = 0


class PaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        name = _lib.pa_status_str(status).decode()
        detail = _lib.pa_last_error().decode()
        super().__init__(f"{fn}: {name}: {detail}")


def _check(fn: str, status: int):
    if status != PA_OK:
        raise PaError(fn, status)


def _arg(t, name, dtype=None, device=True):
    """Pointer of a contiguous tensor of the expected dtype (on the GPU unless
    device=False), or None. The library reads raw memory, so a strided view or
    a wrong element type is refused here rather than misread there."""
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr()


def _same_shape(a, b, names):
    if a is not None and b is not None and tuple(a.shape) != tuple(b.shape):
        raise ValueError(f"{names}: shapes {tuple(a.shape)} and {tuple(b.shape)} differ")


_F16, _I32, _I64 = torch.float16, torch.int32, torch.int64


def _rows(t, name, n, fn, ndim=1):
    """The kernels index these arrays by sequence or token: fewer rows than the
    sizes passed to the library would be read past their end, and an index
    vector with extra dimensions would be misread as a flat one."""
    if t is None:
        return
    if t.dim() != ndim:
        raise ValueError(f"{fn}: {name} must have {ndim} dimension(s), got {tuple(t.shape)}")
    if t.shape[0] != n:
        raise ValueError(f"{fn}: {name} needs {n} rows, has {tuple(t.shape)}")


def _dims(t, n, name, fn):
    if t.dim() != n:
        raise ValueError(f"{fn}: {name} must have {n} dimensions, got {tuple(t.shape)}")


def _pools_fit(k_pool, v_pool, D, fn):
    """Both pools [NB, Hkv, B, D] with the head dimension of the query: a pool
    whose rows are shorter than the query's would be read past its end."""
    _dims(k_pool, 4, "k_pool", fn)
    _same_shape(k_pool, v_pool, "k_pool/v_pool")
    if k_pool.shape[3] != D:
        raise ValueError(f"{fn}: pool rows of {k_pool.shape[3]} values do not match the query's "
                         f"head dimension {D}")


def _pairs(t, fn):
    if t.dim() != 2 or t.shape[1] != 2:
        raise ValueError(f"{fn}: block_mapping must be [n, 2], got {tuple(t.shape)}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def lib() -> ctypes.CDLL:
    return _lib


def pa_version() -> int:
    return _lib.pa_version()


def pa_debug_bounds_selftest() -> int:
    """Debug library: counts one refusal at every site in each source file's
    counters; returns how many files (-1 in the release library)."""
    return _lib.pa_debug_bounds_selftest()


def pa_debug_bounds_violations():
    """Accesses the bounds-checked library refused since the last call, per
    check site ({site name: count}), then reset; None from the release library,
    which has no checks."""
    counts = (ctypes.c_uint * 16)()
    n = _lib.pa_debug_bounds_violations(counts, 16)
    if n == -1:
        return None
    if n < 0:
        raise RuntimeError("pa_debug_bounds_violations: HIP error")
    return {_lib.pa_debug_bounds_site(i).decode(): int(counts[i]) for i in range(n)}


def pa_slot_mapping(block_tables, block_size: int, num_blocks: int, context_lens=None,
                    seq_ids=None, positions=None, out=None, stream=None):
    """int64 slots for new tokens (see pa_slot_mapping in include/pa.h)."""
    _dims(block_tables, 2, "block_tables", "pa_slot_mapping")
    S, MB = block_tables.shape
    T = positions.shape[0] if positions is not None else (
        seq_ids.shape[0] if seq_ids is not None else S)
    _rows(seq_ids, "seq_ids", T, "pa_slot_mapping")
    _rows(positions, "positions", T, "pa_slot_mapping")
    _rows(context_lens, "context_lens", S, "pa_slot_mapping")
    _rows(out, "out", T, "pa_slot_mapping")
    if out is None:
        out = torch.empty(T, dtype=torch.int64, device=block_tables.device)
    _check("pa_slot_mapping", _lib.pa_slot_mapping(
        _arg(out, "out", _I64), _arg(block_tables, "block_tables", _I32),
        _arg(seq_ids, "seq_ids", _I32), _arg(positions, "positions", _I32),
        _arg(context_lens, "context_lens", _I32), T, S, MB, block_size, num_blocks,
        _stream(stream)))
    return out


def pa_write_kv(key, value, k_pool, v_pool, slot_mapping, stream=None):
    """Scatter key/value [T, Hkv, D] into the pools [NB, Hkv, B, D] at their slots."""
    _dims(key, 3, "key", "pa_write_kv")
    _dims(k_pool, 4, "k_pool", "pa_write_kv")
    T, Hkv, D = key.shape
    NB, _, B, _ = k_pool.shape
    _same_shape(key, value, "key/value")
    _same_shape(k_pool, v_pool, "k_pool/v_pool")
    _rows(slot_mapping, "slot_mapping", T, "pa_write_kv")
    if tuple(k_pool.shape[1:2]) != (Hkv,) or k_pool.shape[3] != D:
        raise ValueError(f"pa_write_kv: key {tuple(key.shape)} does not fit pool blocks {tuple(k_pool.shape)}")
    _check("pa_write_kv", _lib.pa_write_kv(
        _arg(key, "key", _F16), _arg(value, "value", _F16), _arg(k_pool, "k_pool", _F16),
        _arg(v_pool, "v_pool", _F16), _arg(slot_mapping, "slot_mapping", _I64),
        T, Hkv, D, B, NB, _stream(stream)))


def pa_append_kv(key, value, k_pool, v_pool, block_tables, context_lens=None, seq_ids=None,
                 positions=None, slot_mapping=None, stream=None):
    """pa_slot_mapping and pa_write_kv in one launch: each new token's key/value
    [T, Hkv, D] goes into its slot found through block_tables; the slots are
    also written to slot_mapping when it is given (int64 [T])."""
    _dims(key, 3, "key", "pa_append_kv")
    _dims(block_tables, 2, "block_tables", "pa_append_kv")
    T, Hkv, D = key.shape
    S, MB = block_tables.shape
    _dims(k_pool, 4, "k_pool", "pa_append_kv")
    NB, _, B, _ = k_pool.shape
    _same_shape(key, value, "key/value")
    _same_shape(k_pool, v_pool, "k_pool/v_pool")
    if tuple(k_pool.shape[1:2]) != (Hkv,) or k_pool.shape[3] != D:
        raise ValueError(f"pa_append_kv: key {tuple(key.shape)} does not fit pool blocks {tuple(k_pool.shape)}")
    _rows(seq_ids, "seq_ids", T, "pa_append_kv")
    _rows(positions, "positions", T, "pa_append_kv")
    _rows(context_lens, "context_lens", S, "pa_append_kv")
    _rows(slot_mapping, "slot_mapping", T, "pa_append_kv")
    _check("pa_append_kv", _lib.pa_append_kv(
        _arg(slot_mapping, "slot_mapping", _I64), _arg(key, "key", _F16),
        _arg(value, "value", _F16), _arg(k_pool, "k_pool", _F16), _arg(v_pool, "v_pool", _F16),
        _arg(block_tables, "block_tables", _I32), _arg(seq_ids, "seq_ids", _I32),
        _arg(positions, "positions", _I32), _arg(context_lens, "context_lens", _I32),
        T, S, MB, Hkv, D, B, NB, _stream(stream)))
    return slot_mapping


def pa_copy_blocks(k_pool, v_pool, block_mapping, stream=None):
    """Copy whole blocks src -> dst for each row of block_mapping [n, 2] (int32)."""
    _dims(k_pool, 4, "k_pool", "pa_copy_blocks")
    NB, Hkv, B, D = k_pool.shape
    _pairs(block_mapping, "pa_copy_blocks")
    n = block_mapping.shape[0]
    _same_shape(k_pool, v_pool, "k_pool/v_pool")
    _check("pa_copy_blocks", _lib.pa_copy_blocks(
        _arg(k_pool, "k_pool", _F16), _arg(v_pool, "v_pool", _F16),
        _arg(block_mapping, "block_mapping", _I32), n, Hkv, D, B, NB, _stream(stream)))


def pa_swap_blocks(dst_k_pool, dst_v_pool, src_k_pool, src_v_pool, block_mapping, stream=None):
    """Copy block src of the source pools to block dst of the destination pools for each row
    (src, dst) of block_mapping [n, 2] (int32, on the device). Pools are device tensors or
    pinned host tensors (pin_memory=True)."""
    _dims(src_k_pool, 4, "src_k_pool", "pa_swap_blocks")
    _dims(dst_k_pool, 4, "dst_k_pool", "pa_swap_blocks")
    NB_src, Hkv, B, D = src_k_pool.shape
    NB_dst = dst_k_pool.shape[0]
    _pairs(block_mapping, "pa_swap_blocks")
    n = block_mapping.shape[0]
    _same_shape(dst_k_pool, dst_v_pool, "dst pools")
    _same_shape(src_k_pool, src_v_pool, "src pools")
    if tuple(dst_k_pool.shape[1:]) != tuple(src_k_pool.shape[1:]):
        raise ValueError("pa_swap_blocks: source and destination blocks differ in shape")
    _check("pa_swap_blocks", _lib.pa_swap_blocks(
        _arg(dst_k_pool, "dst_k_pool", _F16, device=False),
        _arg(dst_v_pool, "dst_v_pool", _F16, device=False),
        _arg(src_k_pool, "src_k_pool", _F16, device=False),
        _arg(src_v_pool, "src_v_pool", _F16, device=False),
        _arg(block_mapping, "block_mapping", _I32, device=False), n, Hkv, D, B, NB_dst, NB_src,
        _stream(stream)))


def pa_decode_partition_size(S, Hq, Hkv, B, max_context_len, partition_size=0) -> int:
    return _lib.pa_decode_partition_size(S, Hq, Hkv, B, max_context_len, partition_size)


def pa_decode_workspace_bytes(S, Hq, Hkv, D, B, max_context_len, partition_size=0) -> int:
    return _lib.pa_decode_workspace_bytes(S, Hq, Hkv, D, B, max_context_len, partition_size)


def pa_decode(query, k_pool, v_pool, block_tables, context_lens, max_context_len: int,
              scale: float, partition_size: int = 0, out=None, workspace=None, stream=None):
    """Paged decode attention; returns out fp16 [S, Hq, D]."""
    _dims(query, 3, "query", "pa_decode")
    _dims(block_tables, 2, "block_tables", "pa_decode")
    S, Hq, D = query.shape
    _pools_fit(k_pool, v_pool, D, "pa_decode")
    NB, Hkv, B, _ = k_pool.shape
    MB = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(query)
    need = pa_decode_workspace_bytes(S, Hq, Hkv, D, B, max_context_len, partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _same_shape(out, query, "out/query")
    _same_shape(k_pool, v_pool, "k_pool/v_pool")
    _rows(block_tables, "block_tables", S, "pa_decode", ndim=2)
    _rows(context_lens, "context_lens", S, "pa_decode")
    _check("pa_decode", _lib.pa_decode(
        _arg(out, "out", _F16), _arg(query, "query", _F16), _arg(k_pool, "k_pool", _F16),
        _arg(v_pool, "v_pool", _F16), _arg(block_tables, "block_tables", _I32),
        _arg(context_lens, "context_lens", _I32), S, Hq, Hkv, D, B, NB, MB,
        int(max_context_len), float(scale), int(partition_size), _arg(workspace, "workspace"),
        ws_bytes, _stream(stream)))
    return out


def pa_decode_static_scratch_bytes() -> int:
    return _lib.pa_decode_static_scratch_bytes()


def pa_decode_static(query, k_pool, v_pool, block_tables, context_lens, max_context_len: int,
                     scale: float, partition_size: int = 0, out=None, stream=None):
    """pa_decode with the partials in the library's per-GPU scratch array
    instead of a workspace (the C call allocates nothing; `out` is allocated
    here only when not passed). Calls that overlap on one GPU race."""
    _dims(query, 3, "query", "pa_decode_static")
    _dims(block_tables, 2, "block_tables", "pa_decode_static")
    S, Hq, D = query.shape
    _pools_fit(k_pool, v_pool, D, "pa_decode_static")
    NB, Hkv, B, _ = k_pool.shape
    MB = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(query)
    _same_shape(out, query, "out/query")
    _rows(block_tables, "block_tables", S, "pa_decode_static", ndim=2)
    _rows(context_lens, "context_lens", S, "pa_decode_static")
    _check("pa_decode_static", _lib.pa_decode_static(
        _arg(out, "out", _F16), _arg(query, "query", _F16), _arg(k_pool, "k_pool", _F16),
        _arg(v_pool, "v_pool", _F16), _arg(block_tables, "block_tables", _I32),
        _arg(context_lens, "context_lens", _I32), S, Hq, Hkv, D, B, NB, MB,
        int(max_context_len), float(scale), int(partition_size), _stream(stream)))
    return out


def pa_prefill(query, k_pool, v_pool, block_tables, context_lens, query_start,
               max_query_len: int, scale: float, out=None, stream=None):
    """Paged causal prefill attention of packed new tokens; returns out fp16 [T, Hq, D]."""
    _dims(query, 3, "query", "pa_prefill")
    _dims(block_tables, 2, "block_tables", "pa_prefill")
    T, Hq, D = query.shape
    _pools_fit(k_pool, v_pool, D, "pa_prefill")
    NB, Hkv, B, _ = k_pool.shape
    S, MB = block_tables.shape
    if out is None:
        out = torch.empty_like(query)
    _same_shape(out, query, "out/query")
    _same_shape(k_pool, v_pool, "k_pool/v_pool")
    if context_lens.dim() != 1 or query_start.dim() != 1 or context_lens.shape[0] != S or \
            query_start.shape[0] != S + 1:
        raise ValueError("pa_prefill: context_lens needs S entries and query_start S + 1")
    _check("pa_prefill", _lib.pa_prefill(
        _arg(out, "out", _F16), _arg(query, "query", _F16), _arg(k_pool, "k_pool", _F16),
        _arg(v_pool, "v_pool", _F16), _arg(block_tables, "block_tables", _I32),
        _arg(context_lens, "context_lens", _I32), _arg(query_start, "query_start", _I32),
        S, T, Hq, Hkv, D, B, NB, MB, int(max_query_len), float(scale), _stream(stream)))
    return out


def pa_stream_read(buffer, sink, workgroups: int = 4096, nbytes: int = None, stream=None):
    """Read-bandwidth probe: one linear pass over a device tensor (measurement utility)."""
    size = buffer.numel() * buffer.element_size()
    n = size if nbytes is None else int(nbytes)
    if not 0 <= n <= size:
        raise ValueError(f"pa_stream_read: nbytes={n} outside the buffer's {size} bytes")
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("pa_stream_read: sink needs 4 bytes")
    _check("pa_stream_read", _lib.pa_stream_read(_arg(buffer, "buffer"), n - n % 16,
                                                 _arg(sink, "sink"), int(workgroups),
                                                 _stream(stream)))


# ---------------------------------------------------------------------------
# Host block manager (host numpy arrays; see the pa_bm_* calls in include/pa.h)
# ---------------------------------------------------------------------------

import numpy as _np


def _np_ptr(a):
    return None if a is None else a.ctypes.data


def _seq_ids(seq_ids, fn):
    """Sequence ids as a contiguous int32 vector: the library reads n ints."""
    ids = _np.ascontiguousarray(seq_ids, dtype=_np.int32)
    if ids.ndim != 1:
        raise ValueError(f"{fn}: seq_ids must be a 1-D list of ids, got shape {ids.shape}")
    return ids


class BlockManager:
    """Owner of one native pa_block_manager; every method is one pa_bm_* call."""

    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int = 0):
        h = _p()
        _check("pa_bm_create", _lib.pa_bm_create(num_blocks, block_size, max_blocks_per_seq,
                                                 ctypes.byref(h)))
        self._h = h
        self.block_size = block_size

    def close(self):
        if self._h:
            _lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_sequence(self) -> int:
        out = _i()
        _check("pa_bm_add_sequence", _lib.pa_bm_add_sequence(self._h, ctypes.byref(out)))
        return out.value

    def fork(self, parent: int) -> int:
        out = _i()
        _check("pa_bm_fork", _lib.pa_bm_fork(self._h, parent, ctypes.byref(out)))
        return out.value

    def append_tokens(self, seq_ids):
        """One token per listed sequence. Returns (slots int64 [n], copy pairs int32 [k, 2]).
        Raises PaError (with .n_applied) when the pool is exhausted mid-batch."""
        ids = _seq_ids(seq_ids, "append_tokens")
        n = len(ids)
        slots = _np.empty(n, dtype=_np.int64)
        pairs = _np.empty((max(n, 1), 2), dtype=_np.int32)
        nc, na = _i(), _i()
        st = _lib.pa_bm_append_tokens(self._h, _np_ptr(ids), n, _np_ptr(slots), _np_ptr(pairs), n,
                                      ctypes.byref(nc), ctypes.byref(na))
        if st != PA_OK:
            err = PaError("pa_bm_append_tokens", st)
            err.n_applied = na.value
            err.slots = slots[:na.value].copy()
            err.copy_pairs = pairs[:nc.value].copy()
            raise err
        return slots, pairs[:nc.value].copy()

    def release(self, seq_id: int) -> int:
        out = _i()
        _check("pa_bm_release", _lib.pa_bm_release(self._h, seq_id, ctypes.byref(out)))
        return out.value

    def table(self, seq_id: int):
        """(block ids int32 [n], number of tokens)."""
        nb, nt = _i(), ctypes.c_int64()
        _check("pa_bm_get_table", _lib.pa_bm_get_table(self._h, seq_id, None, 0, ctypes.byref(nb),
                                                        ctypes.byref(nt)))
        row = _np.empty(max(nb.value, 1), dtype=_np.int32)
        _check("pa_bm_get_table", _lib.pa_bm_get_table(self._h, seq_id, _np_ptr(row), len(row),
                                                        ctypes.byref(nb), ctypes.byref(nt)))
        return row[:nb.value].copy(), nt.value

    def export(self, seq_ids, MB: int):
        """pa_decode inputs for a batch: (block_tables int32 [n, MB], context_lens int32 [n])."""
        ids = _seq_ids(seq_ids, "export")
        tables = _np.empty((len(ids), MB), dtype=_np.int32)
        lens = _np.empty(len(ids), dtype=_np.int32)
        _check("pa_bm_export", _lib.pa_bm_export(self._h, _np_ptr(ids), len(ids), _np_ptr(tables),
                                                 MB, _np_ptr(lens)))
        return tables, lens

    def num_free(self) -> int:
        return _lib.pa_bm_num_free(self._h)

    def refcount(self, block: int) -> int:
        return _lib.pa_bm_refcount(self._h, block)


__all__ = ["PaError", "lib", "LIB_PATH", "pa_version", "pa_slot_mapping", "pa_write_kv",
           "pa_copy_blocks", "pa_decode_partition_size", "pa_decode_workspace_bytes",
           "pa_decode", "pa_decode_static", "pa_decode_static_scratch_bytes", "pa_prefill",
           "pa_swap_blocks", "pa_stream_read", "BlockManager"]
