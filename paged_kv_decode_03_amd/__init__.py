"""Paged-attention decode for MI355X (gfx950): Python binding of libpa.so.

Argument marshalling only: every step of the decode path runs in the HIP
kernels of ``libpa.so`` (built by ``python paged_kv_decode_03_amd/build.py``).
Torch tensors supply device memory and the current stream; the functions
check dtype, device, shape and contiguity, then call the C ABI declared in
``include/pa.h`` with raw pointers. There is no fallback: if the library is
missing, importing this package raises.

Entry points (same names as the C ABI without the ``pa_`` prefix):
  write_kv_cache           slot-mapped write of new K/V (copy or int8)
  decode                   paged decode attention (one pass or split-K partials)
  decode_splitk_reduce     log-sum-exp reduce of split-K partials
  decode_balanced          work-balanced split-K decode with the reduce fused in
  write_decode_balanced    the new-token write and decode_balanced in one call
  write_decode_balanced_noalloc
                           the same, with the workspace in the library's static
                           per-GPU array (no allocation; calls on one GPU must
                           not overlap)
  copy_blocks              copy-on-write copy of whole blocks (K, V, int8 scales)
plus ``workspace`` / ``balanced_workspace`` (allocate with torch) and
``paged_attention`` (decode into a new output tensor, any schedule).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python paged_kv_decode_03_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)
_p, _i, _i64, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
_lib.pa_version.restype = _i
_lib.pa_status_string.restype = ctypes.c_char_p
_lib.pa_status_string.argtypes = [_i]
_lib.pa_num_partitions.restype = _i
_lib.pa_num_partitions.argtypes = [_i, _i]
_lib.pa_write_kv_cache.restype = _i
_lib.pa_write_kv_cache.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i64, _i, _i, _p]
_lib.pa_decode.restype = _i
_lib.pa_decode.argtypes = [_p, _p, _p, _p, _p, _i, _p, _p, _p, _f, _i, _i, _i, _i, _i, _i64, _i,
                           _i, _p, _p, _p, _i, _i, _p]
_lib.pa_decode_balanced.restype = _i
_lib.pa_decode_balanced.argtypes = [_p, _p, _p, _p, _p, _i, _p, _p, _p, _f, _i, _i, _i, _i, _i,
                                    _i64, _i, _i, _p, _p, _p, _p, _i, _i, _p]
_lib.pa_write_decode_balanced.restype = _i
_lib.pa_write_decode_balanced.argtypes = [_p, _p, _p] + _lib.pa_decode_balanced.argtypes
_lib.pa_write_decode_balanced_noalloc.restype = _i
_lib.pa_write_decode_balanced_noalloc.argtypes = (_lib.pa_write_decode_balanced.argtypes[:-7]
                                                  + [_i, _i, _p])
_lib.pa_balanced_workspace.restype = _i
_lib.pa_balanced_workspace.argtypes = [_i, _i, _i, _i, _p, ctypes.POINTER(_i64),
                                       ctypes.POINTER(_i64)]
_lib.pa_copy_blocks.restype = _i
_lib.pa_copy_blocks.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i64, _i, _p]
_lib.pa_decode_splitk_reduce.restype = _i
_lib.pa_prefill.argtypes = [_p, _p, _p, _p, _p, _i, _p, _p, _p, _p, _f, _i, _i, _i, _i, _i, _i,
                            _i, _i64, _i, _i, _p, _p, _p, _p, _i, _i, _p]
_lib.pa_prefill.restype = _i
_lib.pa_write_prefill.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _i, _p, _p, _p, _p, _f, _i, _i,
                                  _i, _i, _i, _i, _i, _i64, _i, _i, _p, _p, _p, _p, _i, _i, _p]
_lib.pa_write_prefill.restype = _i
_lib.pa_decode_splitk_reduce.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p]

PA_F32, PA_BF16, PA_I8 = 0, 1, 2
_DTYPE = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.int8: PA_I8}


class PAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    return _lib


def version() -> int:
    return _lib.pa_version()


def status_string(status: int) -> str:
    return _lib.pa_status_string(int(status)).decode()


def num_partitions(max_context_len: int, partition_size: int) -> int:
    return _lib.pa_num_partitions(int(max_context_len), int(partition_size))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dt(t) -> int:
    try:
        return _DTYPE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, rc):
    if rc != 0:
        raise PAError(fn, rc)


def write_kv_cache(key, value, k_cache, v_cache, slot_mapping, k_scale=None, v_scale=None,
                   stream=None):
    """Write key/value [T, Hkv, D] into the slots ``slot_mapping`` [T] (int64)
    of the pool k_cache/v_cache [NB, Hkv, B, D]; int8 pools need k_scale and
    v_scale [NB, Hkv] fp32."""
    dev = _dev(key, value, k_cache, v_cache, slot_mapping, k_scale, v_scale)
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    T, Hkv, D = key.shape
    NB, Hkv2, B, D2 = k_cache.shape
    if value.shape != key.shape or v_cache.shape != k_cache.shape or (Hkv2, D2) != (Hkv, D) \
            or slot_mapping.shape != (T,):
        raise ValueError("shape mismatch")
    rc = _lib.pa_write_kv_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                _ptr(slot_mapping), _ptr(k_scale), _ptr(v_scale), T, Hkv, D, B,
                                NB, _dt(key), _dt(k_cache), _stream(stream, dev))
    _check("pa_write_kv_cache", rc)


def decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
           partition_size=0, tmp_out=None, tmp_max=None, tmp_sum=None, k_scale=None,
           v_scale=None, stream=None):
    """Paged decode attention of q [S, Hq, D] over the pool; one pass into
    ``out`` [S, Hq, D] (partition_size 0) or split-K partials into the
    workspace (partition_size > 0, a multiple of the block size)."""
    dev = _dev(out, q, k_cache, v_cache, block_tables, context_lens, tmp_out, tmp_max, tmp_sum,
               k_scale, v_scale)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or block_tables.shape[0] != S \
            or context_lens.shape != (S,) or (out is not None and out.shape != q.shape):
        raise ValueError("shape mismatch")
    if out is not None and out.dtype != q.dtype:
        raise TypeError("out must have the dtype of q")
    rc = _lib.pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                        block_tables.shape[1], _ptr(context_lens), _ptr(k_scale), _ptr(v_scale),
                        float(scale), S, Hq, Hkv, D, B, NB, int(max_context_len),
                        int(partition_size), _ptr(tmp_out), _ptr(tmp_max), _ptr(tmp_sum),
                        _dt(q), _dt(k_cache), _stream(stream, dev))
    _check("pa_decode", rc)


def prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale,
            max_query_len, max_context_len, k_scale=None, v_scale=None, partition_size=0,
            tmp_out=None, tmp_max=None, tmp_sum=None, row_lens=None, stream=None):
    """Causal attention of several new query tokens per sequence over the pool:
    q and out [T, Hq, D]; rows query_start_loc[s] .. [s+1]-1 are the newest
    tokens of sequence s (already written to the cache and counted by
    context_lens). partition_size > 0: split-K partials into the workspace
    (``prefill_workspace``) instead of ``out``; combine them with
    ``decode_splitk_reduce(out, tmp_out, tmp_max, tmp_sum, row_lens, ...)``."""
    dev = _dev(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc, k_scale,
               v_scale, tmp_out, tmp_max, tmp_sum, row_lens)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 \
            or query_start_loc.dtype != torch.int32:
        raise TypeError("block_tables, context_lens and query_start_loc must be int32")
    T, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    S = context_lens.shape[0]
    if D2 != D or v_cache.shape != k_cache.shape or block_tables.shape[0] != S \
            or query_start_loc.shape != (S + 1,) or (out is not None and out.shape != q.shape):
        raise ValueError("shape mismatch")
    if out is not None and out.dtype != q.dtype:
        raise TypeError("out must have the dtype of q")
    rc = _lib.pa_prefill(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                         block_tables.shape[1], _ptr(context_lens), _ptr(query_start_loc),
                         _ptr(k_scale), _ptr(v_scale), float(scale), S, T, int(max_query_len),
                         Hq, Hkv, D, B, NB, int(max_context_len), int(partition_size),
                         _ptr(tmp_out), _ptr(tmp_max), _ptr(tmp_sum), _ptr(row_lens), _dt(q),
                         _dt(k_cache), _stream(stream, dev))
    _check("pa_prefill", rc)


def write_prefill(key, value, slot_mapping, out, q, k_cache, v_cache, block_tables,
                  context_lens, query_start_loc, scale, max_query_len, max_context_len,
                  k_scale=None, v_scale=None, partition_size=0, tmp_out=None, tmp_max=None,
                  tmp_sum=None, row_lens=None, stream=None):
    """pa_write_kv_cache of the new tokens (key / value [T, Hkv, D] bf16, one row
    per query row, slot_mapping [T] int64) and pa_prefill in one launch; a bf16
    or int8 cache (k_scale / v_scale [NB, Hkv] fp32 for int8)."""
    dev = _dev(key, value, slot_mapping, out, q, k_cache, v_cache, block_tables, context_lens,
               query_start_loc, k_scale, v_scale, tmp_out, tmp_max, tmp_sum, row_lens)
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    T, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    S = context_lens.shape[0]
    if key.shape != (T, Hkv, D) or value.shape != key.shape or slot_mapping.shape != (T,) \
            or D2 != D or v_cache.shape != k_cache.shape or block_tables.shape[0] != S \
            or query_start_loc.shape != (S + 1,) or (out is not None and out.shape != q.shape):
        raise ValueError("shape mismatch")
    rc = _lib.pa_write_prefill(_ptr(key), _ptr(value), _ptr(slot_mapping), _ptr(out), _ptr(q),
                               _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                               block_tables.shape[1], _ptr(context_lens), _ptr(query_start_loc),
                               _ptr(k_scale), _ptr(v_scale), float(scale), S, T, int(max_query_len), Hq, Hkv, D, B, NB,
                               int(max_context_len), int(partition_size), _ptr(tmp_out),
                               _ptr(tmp_max), _ptr(tmp_sum), _ptr(row_lens), _dt(q),
                               _dt(k_cache), _stream(stream, dev))
    _check("pa_write_prefill", rc)


def prefill_workspace(num_query_tokens, num_heads, head_dim, max_context_len, partition_size,
                      device):
    """(tmp_out, tmp_max, tmp_sum, row_lens) for pa_prefill's split-K."""
    NP = max(1, num_partitions(max_context_len, partition_size))
    T, H, D = num_query_tokens, num_heads, head_dim
    return (torch.empty((T, H, NP, D), dtype=torch.float32, device=device),
            torch.empty((T, H, NP), dtype=torch.float32, device=device),
            torch.empty((T, H, NP), dtype=torch.float32, device=device),
            torch.empty((T,), dtype=torch.int32, device=device))


def decode_splitk_reduce(out, tmp_out, tmp_max, tmp_sum, context_lens, max_context_len,
                         partition_size, stream=None):
    """Combine split-K partials [S, Hq, NP, D] into out [S, Hq, D]."""
    dev = _dev(out, tmp_out, tmp_max, tmp_sum, context_lens)
    S, Hq, D = out.shape
    rc = _lib.pa_decode_splitk_reduce(_ptr(out), _ptr(tmp_out), _ptr(tmp_max), _ptr(tmp_sum),
                                      _ptr(context_lens), S, Hq, D, int(max_context_len),
                                      int(partition_size), _dt(out), _stream(stream, dev))
    _check("pa_decode_splitk_reduce", rc)


def copy_blocks(k_cache, v_cache, block_mapping, k_scale=None, v_scale=None, stream=None):
    """Copy every byte of block block_mapping[i, 0] into block block_mapping[i, 1]
    of both pools (and of the int8 scales); block_mapping [n, 2] int64 on the
    device, destinations distinct and never a source."""
    dev = _dev(k_cache, v_cache, block_mapping, k_scale, v_scale)
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 \
            or block_mapping.shape[1] != 2:
        raise TypeError("block_mapping must be int64 [n, 2]")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    NB, Hkv, B, D = k_cache.shape
    if k_cache.dtype == torch.int8:
        if k_scale is None or v_scale is None or k_scale.shape != (NB, Hkv) \
                or v_scale.shape != (NB, Hkv) or k_scale.dtype != torch.float32 \
                or v_scale.dtype != torch.float32:
            raise ValueError("an int8 pool needs fp32 k_scale and v_scale [NB, Hkv]")
    rc = _lib.pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                             _ptr(block_mapping), block_mapping.shape[0], Hkv, D, B, NB,
                             _dt(k_cache), _stream(stream, dev))
    _check("pa_copy_blocks", rc)


def balanced_sizes(num_seqs, num_heads, num_kv_heads, head_dim, device=None):
    """(slots, counters) of the balanced schedule's workspace on ``device``
    (pa_balanced_workspace): tmp_out [slots, G, D], tmp_max / tmp_sum
    [slots, G] fp32, counters int32 [counters]."""
    dev = torch.device("cuda" if device is None else device)
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    slots, counters = _i64(0), _i64(0)
    rc = _lib.pa_balanced_workspace(int(num_seqs), int(num_heads), int(num_kv_heads),
                                    int(head_dim), _stream(None, dev), ctypes.byref(slots),
                                    ctypes.byref(counters))
    _check("pa_balanced_workspace", rc)
    return slots.value, counters.value


def _check_balanced_ws(q, num_kv_heads, tmp_out, tmp_max, tmp_sum, counters):
    S, Hq, D = q.shape
    ns, nc = balanced_sizes(S, Hq, num_kv_heads, D, q.device)
    G = Hq // num_kv_heads
    if tmp_out.numel() < ns * G * D or tmp_max.numel() < ns * G or tmp_sum.numel() < ns * G \
            or counters.numel() < nc:
        raise ValueError("workspace too small (see balanced_sizes)")


def decode_balanced(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                    max_context_len, min_piece_tokens, tmp_out, tmp_max, tmp_sum, counters,
                    k_scale=None, v_scale=None, stream=None):
    """Work-balanced decode into ``out`` [S, Hq, D]; ``counters`` [S, Hkv] int32
    must be zero on entry and is zero again on return."""
    dev = _dev(out, q, k_cache, v_cache, block_tables, context_lens, tmp_out, tmp_max, tmp_sum,
               counters, k_scale, v_scale)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 \
            or counters.dtype != torch.int32:
        raise TypeError("block_tables, context_lens and counters must be int32")
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or block_tables.shape[0] != S \
            or context_lens.shape != (S,) or out.shape != q.shape:
        raise ValueError("shape mismatch")
    _check_balanced_ws(q, Hkv, tmp_out, tmp_max, tmp_sum, counters)
    if out.dtype != q.dtype:
        raise TypeError("out must have the dtype of q")
    rc = _lib.pa_decode_balanced(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                 _ptr(k_scale), _ptr(v_scale), float(scale), S, Hq, Hkv, D, B, NB,
                                 int(max_context_len), int(min_piece_tokens), _ptr(tmp_out),
                                 _ptr(tmp_max), _ptr(tmp_sum), _ptr(counters), _dt(q),
                                 _dt(k_cache), _stream(stream, dev))
    _check("pa_decode_balanced", rc)


def write_decode_balanced(key, value, slot_mapping, out, q, k_cache, v_cache, block_tables,
                          context_lens, scale, max_context_len, min_piece_tokens, tmp_out,
                          tmp_max, tmp_sum, counters, k_scale=None, v_scale=None, stream=None):
    """write_kv_cache(key, value, k_cache, v_cache, slot_mapping) followed by
    decode_balanced, in one call (one launch where the kernel supports it):
    key/value [S, Hkv, D] hold each sequence's new token, slot_mapping [S]
    (int64) its slot at logical position context_lens[s] - 1."""
    dev = _dev(key, value, slot_mapping, out, q, k_cache, v_cache, block_tables, context_lens,
               tmp_out, tmp_max, tmp_sum, counters, k_scale, v_scale)
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 \
            or counters.dtype != torch.int32:
        raise TypeError("block_tables, context_lens and counters must be int32")
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    if key.shape != (S, Hkv, D) or value.shape != key.shape or slot_mapping.shape != (S,) \
            or key.dtype != q.dtype or value.dtype != q.dtype:
        raise ValueError("key/value must be [S, Hkv, D] of q's dtype, slot_mapping [S]")
    if D2 != D or v_cache.shape != k_cache.shape or block_tables.shape[0] != S \
            or context_lens.shape != (S,) or out.shape != q.shape:
        raise ValueError("shape mismatch")
    _check_balanced_ws(q, Hkv, tmp_out, tmp_max, tmp_sum, counters)
    if out.dtype != q.dtype:
        raise TypeError("out must have the dtype of q")
    rc = _lib.pa_write_decode_balanced(_ptr(key), _ptr(value), _ptr(slot_mapping), _ptr(out),
                                       _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                       block_tables.shape[1], _ptr(context_lens), _ptr(k_scale),
                                       _ptr(v_scale), float(scale), S, Hq, Hkv, D, B, NB,
                                       int(max_context_len), int(min_piece_tokens),
                                       _ptr(tmp_out), _ptr(tmp_max), _ptr(tmp_sum),
                                       _ptr(counters), _dt(q), _dt(k_cache),
                                       _stream(stream, dev))
    _check("pa_write_decode_balanced", rc)


def write_decode_balanced_noalloc(key, value, slot_mapping, out, q, k_cache, v_cache,
                                  block_tables, context_lens, scale, max_context_len,
                                  min_piece_tokens, k_scale=None, v_scale=None, stream=None):
    """write_decode_balanced with the workspace in the library's static array:
    nothing is allocated. Shapes whose workspace does not fit that array raise
    PAError (shape); calls that overlap in time on one GPU race."""
    dev = _dev(key, value, slot_mapping, out, q, k_cache, v_cache, block_tables, context_lens,
               k_scale, v_scale)
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    if key.shape != (S, Hkv, D) or value.shape != key.shape or slot_mapping.shape != (S,) \
            or key.dtype != q.dtype or value.dtype != q.dtype:
        raise ValueError("key/value must be [S, Hkv, D] of q's dtype, slot_mapping [S]")
    if D2 != D or v_cache.shape != k_cache.shape or block_tables.shape[0] != S \
            or context_lens.shape != (S,) or out.shape != q.shape:
        raise ValueError("shape mismatch")
    if out.dtype != q.dtype:
        raise TypeError("out must have the dtype of q")
    rc = _lib.pa_write_decode_balanced_noalloc(
        _ptr(key), _ptr(value), _ptr(slot_mapping), _ptr(out), _ptr(q), _ptr(k_cache),
        _ptr(v_cache), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        _ptr(k_scale), _ptr(v_scale), float(scale), S, Hq, Hkv, D, B, NB, int(max_context_len),
        int(min_piece_tokens), _dt(q), _dt(k_cache), _stream(stream, dev))
    _check("pa_write_decode_balanced_noalloc", rc)


def balanced_workspace(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                       min_piece_tokens, device):
    """(tmp_out, tmp_max, tmp_sum, counters) for decode_balanced; counters zeroed.
    The sizes depend on the device and the head shape only (balanced_sizes);
    max_context_len and min_piece_tokens are accepted for symmetry with
    ``workspace`` and do not change them."""
    ns, nc = balanced_sizes(num_seqs, num_heads, num_kv_heads, head_dim, device)
    G = num_heads // num_kv_heads
    return (torch.empty((ns, G, head_dim), dtype=torch.float32, device=device),
            torch.empty((ns, G), dtype=torch.float32, device=device),
            torch.empty((ns, G), dtype=torch.float32, device=device),
            torch.zeros((nc,), dtype=torch.int32, device=device))


def workspace(num_seqs, num_heads, head_dim, max_context_len, partition_size, device):
    """Split-K partials (tmp_out [S,Hq,NP,D], tmp_max, tmp_sum [S,Hq,NP]) fp32."""
    NP = max(1, num_partitions(max_context_len, partition_size))
    return (torch.empty((num_seqs, num_heads, NP, head_dim), dtype=torch.float32, device=device),
            torch.empty((num_seqs, num_heads, NP), dtype=torch.float32, device=device),
            torch.empty((num_seqs, num_heads, NP), dtype=torch.float32, device=device))


def paged_attention(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                    partition_size=0, k_scale=None, v_scale=None, ws=None, stream=None,
                    balanced=False):
    """Decode attention into a new tensor: one pass (partition_size 0), split-K
    partitions + reduce, or (balanced=True) the work-balanced schedule with
    pieces of at least partition_size tokens."""
    out = torch.empty_like(q)
    S, Hq, D = q.shape
    if balanced:
        if ws is None:
            ws = balanced_workspace(S, Hq, k_cache.shape[1], D, max_context_len, partition_size,
                                    q.device)
        decode_balanced(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                        max_context_len, partition_size, *ws, k_scale=k_scale, v_scale=v_scale,
                        stream=stream)
        return out
    if partition_size == 0:
        decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, 0,
               k_scale=k_scale, v_scale=v_scale, stream=stream)
        return out
    if ws is None:
        ws = workspace(S, Hq, D, max_context_len, partition_size, q.device)
    decode(None, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
           partition_size, *ws, k_scale=k_scale, v_scale=v_scale, stream=stream)
    decode_splitk_reduce(out, *ws, context_lens, max_context_len, partition_size, stream=stream)
    return out
