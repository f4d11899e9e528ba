"""ctypes front end of the fp64 paged-attention decode oracle (``oracle.c``).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
bench's ``cpu_baseline`` leg may import this package. The HIP library and its
Python binding never import it, and it imports nothing from them.

All arrays are host numpy arrays. bf16 data travels as uint16 bit patterns,
fp32 as float32, int8 as int8; the oracle widens every stored element exactly
to fp64 and returns fp64 outputs.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_DT = {"f32": 0, "bf16": 1, "i8": 2}
_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_f = ctypes.c_float


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def _dtype_of(a: np.ndarray) -> str:
    return {np.dtype(np.float32): "f32", np.dtype(np.uint16): "bf16", np.dtype(np.int8): "i8"}[a.dtype]


def num_partitions(max_context_len: int, partition_size: int) -> int:
    return -(-int(max_context_len) // int(partition_size))


class Oracle:
    """One loaded build of ``oracle.c`` (the default build, or a test's variant)."""

    def __init__(self, path: str = _LIB_PATH):
        if not os.path.exists(path):
            if path != _LIB_PATH:
                raise FileNotFoundError(path)
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(path)
        lib.ora_write_kv_cache.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i64, _i, _i, _i, _i64, _i, _i]
        lib.ora_decode.argtypes = [_p, _p, _p, _p, _p, _i, _p, _p, _p, _f, _i, _i, _i, _i, _i,
                                   _i64, _i, _i]
        lib.ora_decode_partials.argtypes = [_p, _p, _p, _i, _p, _p, _p, _p, _i, _p, _p, _p, _f,
                                            _i, _i, _i, _i, _i, _i64, _i, _i, _i]
        lib.ora_splitk_reduce.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i]
        lib.ora_prefill.argtypes = [_p, _p, _p, _p, _p, _i, _p, _p, _p, _p, _f, _i, _i, _i, _i,
                                    _i, _i, _i64, _i, _i]
        lib.ora_copy_blocks.argtypes = [_p, _p, _p, _p, _p, _i64, _i, _i, _i, _i64, _i]
        lib.ora_num_threads.restype = _i
        lib.ora_set_num_threads.argtypes = [_i]
        self.lib = lib
        self.path = path

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise OracleError(f"{what} returned {rc}")

    def num_threads(self) -> int:
        return self.lib.ora_num_threads()

    def set_num_threads(self, n: int) -> None:
        self.lib.ora_set_num_threads(int(n))

    def write_kv_cache(self, key, value, k_cache, v_cache, slot_mapping, k_scale=None, v_scale=None):
        """Slot-mapped write into (k_cache, v_cache) [NB, Hkv, B, D], in place."""
        assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
        key, value = _c(key), _c(value)
        slot_mapping = _c(slot_mapping, np.int64)
        k_scale, v_scale = _c(k_scale, np.float32), _c(v_scale, np.float32)
        NB, Hkv, B, D = k_cache.shape
        T = slot_mapping.shape[0]
        assert key.shape == (T, Hkv, D) and value.shape == (T, Hkv, D)
        rc = self.lib.ora_write_kv_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(slot_mapping), _ptr(k_scale), _ptr(v_scale), T, Hkv,
                                         D, B, NB, _DT[_dtype_of(key)], _DT[_dtype_of(k_cache)])
        self._check(rc, "ora_write_kv_cache")

    def copy_blocks(self, k_cache, v_cache, block_mapping, k_scale=None, v_scale=None):
        """Copy-on-write block copy, in place: block_mapping [n, 2] int64 (src, dst).
        int8 pools copy their scales [NB, Hkv] too (pass them as float32 arrays)."""
        assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
        for sc in (k_scale, v_scale):
            assert sc is None or (sc.dtype == np.float32 and sc.flags.c_contiguous)
        mapping = _c(np.asarray(block_mapping).reshape(-1, 2), np.int64)
        NB, Hkv, B, D = k_cache.shape
        rc = self.lib.ora_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                      _ptr(mapping), mapping.shape[0], Hkv, D, B, NB,
                                      _DT[_dtype_of(k_cache)])
        self._check(rc, "ora_copy_blocks")

    def decode(self, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale=None,
               v_scale=None):
        """Paged decode attention in fp64: returns out [S, Hq, D] float64."""
        q = _c(q)
        block_tables, context_lens = _c(block_tables, np.int32), _c(context_lens, np.int32)
        k_scale, v_scale = _c(k_scale, np.float32), _c(v_scale, np.float32)
        S, Hq, D = q.shape
        NB, Hkv, B, D2 = k_cache.shape
        assert D2 == D and block_tables.shape[0] == S and context_lens.shape == (S,)
        out = np.empty((S, Hq, D), dtype=np.float64)
        rc = self.lib.ora_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                 _ptr(k_scale), _ptr(v_scale), float(scale), S, Hq, Hkv, D, B, NB,
                                 _DT[_dtype_of(q)], _DT[_dtype_of(k_cache)])
        self._check(rc, "ora_decode")
        return out

    def prefill(self, q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale,
                k_scale=None, v_scale=None):
        """Several query tokens per sequence (the newest n_s tokens of sequence
        s, rows query_start_loc[s] .. [s+1]-1 of q), causal over the cached
        context: returns out [num_query_tokens, Hq, D] float64."""
        q = _c(q)
        block_tables, context_lens = _c(block_tables, np.int32), _c(context_lens, np.int32)
        query_start_loc = _c(query_start_loc, np.int32)
        k_scale, v_scale = _c(k_scale, np.float32), _c(v_scale, np.float32)
        T, Hq, D = q.shape
        NB, Hkv, B, D2 = k_cache.shape
        S = context_lens.shape[0]
        assert D2 == D and block_tables.shape[0] == S and query_start_loc.shape == (S + 1,)
        out = np.empty((T, Hq, D), dtype=np.float64)
        rc = self.lib.ora_prefill(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                  _ptr(query_start_loc), _ptr(k_scale), _ptr(v_scale),
                                  float(scale), S, T, Hq, Hkv, D, B, NB, _DT[_dtype_of(q)],
                                  _DT[_dtype_of(k_cache)])
        self._check(rc, "ora_prefill")
        return out

    def decode_partials(self, q, k_cache, v_cache, block_tables, context_lens, scale,
                        partition_size, k_scale=None, v_scale=None, num_parts=None):
        """Split-K partials: (o [S,Hq,NP,D], m [S,Hq,NP], l [S,Hq,NP]) float64.
        Entries of partitions past a sequence's length are left as NaN."""
        q = _c(q)
        block_tables, context_lens = _c(block_tables, np.int32), _c(context_lens, np.int32)
        k_scale, v_scale = _c(k_scale, np.float32), _c(v_scale, np.float32)
        S, Hq, D = q.shape
        NB, Hkv, B, _ = k_cache.shape
        NP = num_parts if num_parts is not None else num_partitions(
            context_lens.max() if S else 0, partition_size)
        o = np.full((S, Hq, NP, D), np.nan)
        m = np.full((S, Hq, NP), np.nan)
        l = np.full((S, Hq, NP), np.nan)
        rc = self.lib.ora_decode_partials(
            _ptr(o), _ptr(m), _ptr(l), NP, _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), _ptr(k_scale),
            _ptr(v_scale), float(scale), S, Hq, Hkv, D, B, NB, int(partition_size),
            _DT[_dtype_of(q)], _DT[_dtype_of(k_cache)])
        self._check(rc, "ora_decode_partials")
        return o, m, l

    def splitk_reduce(self, o, m, l, context_lens, partition_size):
        """Log-sum-exp combination of split-K partials -> out [S, Hq, D] float64."""
        o, m, l = _c(o, np.float64), _c(m, np.float64), _c(l, np.float64)
        context_lens = _c(context_lens, np.int32)
        S, Hq, NP, D = o.shape
        out = np.empty((S, Hq, D), dtype=np.float64)
        rc = self.lib.ora_splitk_reduce(_ptr(out), _ptr(o), _ptr(m), _ptr(l), _ptr(context_lens),
                                        S, Hq, D, int(partition_size), NP)
        self._check(rc, "ora_splitk_reduce")
        return out

    def fill_cache(self, case):
        """Pool of a ``synth.Case`` as the oracle's own write leaves it: poison,
        then every token already in context, then the new token of each sequence."""
        k, v = case.empty_pool()
        self.write_kv_cache(case.pre_key, case.pre_value, k, v, case.pre_slots, case.k_scale,
                            case.v_scale)
        self.write_kv_cache(case.key, case.value, k, v, case.slot_mapping, case.k_scale,
                            case.v_scale)
        return k, v

    def decode_case(self, case, k=None, v=None, seqs=None):
        """Oracle decode of a ``synth.Case`` (optionally only sequences ``seqs``)."""
        if k is None:
            k, v = self.fill_cache(case)
        sel = slice(None) if seqs is None else np.asarray(seqs)
        return self.decode(case.q[sel], k, v, case.block_tables[sel], case.context_lens[sel],
                           case.scale, case.k_scale, case.v_scale)


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def num_threads():
    return default().num_threads()


def set_num_threads(n):
    default().set_num_threads(n)


def write_kv_cache(*a, **kw):
    return default().write_kv_cache(*a, **kw)


def decode(*a, **kw):
    return default().decode(*a, **kw)


def prefill(*a, **kw):
    return default().prefill(*a, **kw)


def decode_partials(*a, **kw):
    return default().decode_partials(*a, **kw)


def splitk_reduce(*a, **kw):
    return default().splitk_reduce(*a, **kw)


def copy_blocks(*a, **kw):
    return default().copy_blocks(*a, **kw)


def fill_cache(case):
    return default().fill_cache(case)


def decode_case(case, k=None, v=None, seqs=None):
    return default().decode_case(case, k, v, seqs)
