"""Paged KV-cache attention for MI355X (gfx950): a thin Python binding.

Each function here marshals torch tensors into the C ABI of ``libpa.so``
(declared in ``include/pa.h``) and returns; every step of the computation
runs in the library's HIP kernels, on torch's current stream.  There is no
fallback: if ``libpa.so`` is missing, importing this package raises.

Names follow the C ABI: ``pa_reshape_and_cache``, ``pa_copy_blocks``, ``pa_decode``,
``pa_decode_partitions``, ``pa_decode_merge``, ``pa_decode_multi``, ``pa_prefill_paged``,
``pa_decode_workspace_size``, ``pa_decode_default_partition``,
``pa_kv_bytes_per_token``, ``pa_status_string``, and for an FP8 (E4M3) cache
``pa_reshape_and_cache_fp8``, ``pa_copy_blocks_fp8``, ``pa_decode_fp8``,
``pa_decode_partitions_fp8``, ``pa_prefill_paged_fp8``, and ``pa_decode_noalloc`` for
callers that cannot allocate (its split-KV partials live in a static scratch).

With the environment variable ``PA_DEBUG_BOUNDS=1`` set at import, the package
loads ``libpa_debug.so`` instead: the same kernels, with every call's
device-resident indices checked first; ``pa_debug_bounds`` reads the result.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "PagedKVError", "LIB_PATH", "BLOCK_SIZE", "PA_DECODE_STREAM_KV", "PA_DECODE_SHARED_PREFIX",
    "PA_PARTITION_BALANCED", "lib",
    "pa_kv_bytes_per_token", "pa_status_string", "pa_reshape_and_cache", "pa_copy_blocks",
    "pa_decode_default_partition", "pa_decode_split", "pa_decode_workspace_size", "pa_decode",
    "pa_decode_step", "pa_decode_partitions_step",
    "pa_decode_partitions", "pa_decode_merge", "pa_prefill_paged",
    "pa_reshape_and_cache_fp8", "pa_copy_blocks_fp8", "pa_decode_fp8", "pa_decode_partitions_fp8",
    "pa_prefill_paged_fp8", "pa_decode_multi", "pa_decode_noalloc", "NOALLOC_SCRATCH_BYTES",
    "pa_debug_bounds", "DEBUG_BOUNDS_BITS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "libpa_debug.so" if os.environ.get("PA_DEBUG_BOUNDS") == "1" else "libpa.so")
BLOCK_SIZE = 16
PA_DECODE_STREAM_KV = 1   # no physical block is read twice in the call: stream K/V
PA_DECODE_SHARED_PREFIX = 2   # consecutive sequences may share blocks: read each shared block once per wave
PA_PARTITION_BALANCED = -1   # partition_tokens value: the balanced split of decode work
NOALLOC_SCRATCH_BYTES = 64 << 20   # PA_NOALLOC_SCRATCH_BYTES: static scratch of pa_decode_noalloc
# bits of pa_debug_bounds (PA_DEBUG_* in pa.h)
DEBUG_BOUNDS_BITS = {"block_id": 1, "seq_len": 2, "slot": 4, "query_range": 8}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python paged_kv_cache_24_amd/build.py` "
        "(hipcc for gfx950). There is no non-HIP fallback.")

lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_u32 = ctypes.c_uint32

_SIGS = {
    "pa_kv_bytes_per_token": (ctypes.c_uint64, [_i32, _i32, _i32, _i32]),
    "pa_status_string": (ctypes.c_char_p, [_i32]),
    "pa_reshape_and_cache": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _i32, _vp]),
    "pa_copy_blocks": (_i32, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _i32, _vp]),
    "pa_decode_default_partition": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_split": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64,
                         _f32, _i32, _i32, _u32, _vp, _sz, _vp]),
    "pa_decode_partitions": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                    _i32, _i64, _f32, _i32, _i32, _u32, _vp, _sz, _vp]),
    "pa_decode_step": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                              _i64, _f32, _i32, _i32, _u32, _vp, _sz, _vp]),
    "pa_decode_partitions_step": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                         _i32, _i64, _f32, _i32, _i32, _u32, _vp, _sz, _vp]),
    "pa_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                 _i64, _f32, _i32, _i32, _u32, _vp]),
    "pa_decode_multi": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                               _i64, _f32, _i32, _i32, _u32, _vp, _sz, _vp]),
    "pa_decode_merge": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _sz,
                               _vp]),
    "pa_prefill_paged": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32,
                                _i32, _i32, _i32, _i64, _f32, _i32, _vp]),
    "pa_reshape_and_cache_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
                                        _i64, _i32, _vp]),
    "pa_copy_blocks_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _vp]),
    "pa_prefill_paged_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32,
                                    _i32, _i32, _i32, _i32, _i32, _i64, _f32, _i32, _vp]),
    "pa_decode_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                             _i32, _i64, _f32, _i32, _i32, _u32, _vp, _sz, _vp]),
    "pa_decode_partitions_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                        _i32, _i32, _i32, _i64, _f32, _i32, _i32, _u32, _vp, _sz,
                                        _vp]),
    "pa_debug_bounds": (_i32, [ctypes.POINTER(_u32), _i32, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

_DTYPE = {torch.float16: 0, torch.bfloat16: 1}


class PagedKVError(RuntimeError):
    """A non-zero status from libpa."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({pa_status_string(status)})")


def _check(fn: str, status: int):
    if status != 0:
        raise PagedKVError(fn, status)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t, name, dtype=None, ndim=None, device=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")


def _kv_dtype(cache):
    if cache.dtype not in _DTYPE:
        raise TypeError(f"cache dtype must be float16 or bfloat16, got {cache.dtype}")
    return _DTYPE[cache.dtype]


def pa_kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    return int(lib.pa_kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes))


def pa_status_string(status: int) -> str:
    return lib.pa_status_string(status).decode()


def pa_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None):
    """Store ``key[t]``/``value[t]`` (``[N, Hkv, D]``) at slot ``slot_mapping[t]``
    of ``k_cache``/``v_cache`` (``[NB, 16, Hkv, D]``); negative slots are skipped."""
    _need(k_cache, "k_cache", ndim=4)
    _need(v_cache, "v_cache", k_cache.dtype, 4)
    _need(key, "key", k_cache.dtype, 3)
    _need(value, "value", k_cache.dtype, 3)
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    nb, bs, hkv, d = k_cache.shape
    if v_cache.shape != k_cache.shape or key.shape != value.shape or tuple(key.shape[1:]) != (hkv, d):
        raise ValueError("key/value/cache shapes disagree")
    if slot_mapping.shape[0] != key.shape[0]:
        raise ValueError("slot_mapping needs one entry per token")
    _check("pa_reshape_and_cache", lib.pa_reshape_and_cache(
        _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), key.shape[0],
        hkv, d, bs, nb, _kv_dtype(k_cache), _stream(stream)))


def pa_copy_blocks(k_cache, v_cache, block_pairs, stream=None):
    """Copy whole blocks: ``block_pairs`` is int64 ``[N, 2]`` of (src, dst) rows."""
    _need(k_cache, "k_cache", ndim=4)
    _need(v_cache, "v_cache", k_cache.dtype, 4)
    _need(block_pairs, "block_pairs", torch.int64, 2)
    nb, bs, hkv, d = k_cache.shape
    if v_cache.shape != k_cache.shape or block_pairs.shape[1] != 2:
        raise ValueError("cache shapes disagree or block_pairs is not [N, 2]")
    _check("pa_copy_blocks", lib.pa_copy_blocks(
        _ptr(k_cache), _ptr(v_cache), _ptr(block_pairs), block_pairs.shape[0], hkv, d, bs, nb,
        _kv_dtype(k_cache), _stream(stream)))


def pa_decode_default_partition(num_q_heads: int, num_kv_heads: int, head_dim: int,
                                block_size: int, max_blocks_per_seq: int) -> int:
    return int(lib.pa_decode_default_partition(num_q_heads, num_kv_heads, head_dim, block_size,
                                               max_blocks_per_seq))


def pa_decode_split(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                    partition_tokens=0) -> int:
    """Partition length (tokens) a single-query decode of this shape uses, or
    ``PA_PARTITION_BALANCED`` for the balanced split; 0 for invalid arguments."""
    return int(lib.pa_decode_split(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                   max_blocks_per_seq, partition_tokens))


def pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                             max_blocks_per_seq, partition_tokens=0) -> int:
    return int(lib.pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                            block_size, max_blocks_per_seq, partition_tokens))


def _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens):
    _need(k_cache, "k_cache", ndim=4)
    _need(v_cache, "v_cache", k_cache.dtype, 4)
    _need(q, "q", k_cache.dtype, 3)
    _need(out, "out", k_cache.dtype, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    nb, bs, hkv, d = k_cache.shape
    b, hq, dq = q.shape
    if v_cache.shape != k_cache.shape or out.shape != q.shape or dq != d:
        raise ValueError("q/out/cache shapes disagree")
    if block_tables.shape[0] != b or seq_lens.shape[0] != b:
        raise ValueError("block_tables and seq_lens need one row per sequence")
    return nb, bs, hkv, d, b, hq, block_tables.shape[1]


def _workspace(workspace, need, device):
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    return workspace, workspace.numel() * workspace.element_size()


def pa_decode(out, q, k_cache, v_cache, block_tables, seq_lens, scale, partition_tokens=0,
              workspace=None, stream=None, flags=0):
    """Paged decode attention into ``out`` (``[B, Hq, D]``).  ``workspace`` (bytes,
    see ``pa_decode_workspace_size``) is allocated with torch when not given.
    ``flags``: 0, ``PA_DECODE_STREAM_KV`` (no block shared within the batch) and/or
    ``PA_DECODE_SHARED_PREFIX`` (consecutive sequences may share blocks)."""
    nb, bs, hkv, d, b, hq, mb = _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens)
    need = pa_decode_workspace_size(b, hq, hkv, d, bs, mb, partition_tokens)
    ws, ws_bytes = _workspace(workspace, need, q.device)
    _check("pa_decode", lib.pa_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens), b, hq,
        hkv, d, bs, mb, nb, float(scale), _kv_dtype(k_cache), partition_tokens, flags, _ptr(ws), ws_bytes,
        _stream(stream)))
    return out


def _new_rows(key, value, q, hkv, d):
    _need(key, "key", q.dtype, 3)
    _need(value, "value", q.dtype, 3)
    if tuple(key.shape) != (q.shape[0], hkv, d) or tuple(value.shape) != tuple(key.shape):
        raise ValueError(f"key/value must be [{q.shape[0]}, {hkv}, {d}], got {tuple(key.shape)} / "
                         f"{tuple(value.shape)}")


def pa_decode_step(out, q, key, value, k_cache, v_cache, block_tables, seq_lens, scale, partition_tokens=0,
                   workspace=None, stream=None, flags=0):
    """One decode step: the cache write of each sequence's newest token
    (``key``/``value`` ``[B, Hkv, D]``, position ``seq_lens[b] - 1``) and
    ``pa_decode``, the write done inside the decode kernels."""
    nb, bs, hkv, d, b, hq, mb = _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens)
    _new_rows(key, value, q, hkv, d)
    need = pa_decode_workspace_size(b, hq, hkv, d, bs, mb, partition_tokens)
    ws, ws_bytes = _workspace(workspace, need, q.device)
    _check("pa_decode_step", lib.pa_decode_step(
        _ptr(out), _ptr(q), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(seq_lens), b, hq, hkv, d, bs, mb, nb, float(scale), _kv_dtype(k_cache), partition_tokens, flags,
        _ptr(ws), ws_bytes, _stream(stream)))
    return out


def pa_decode_partitions_step(out, q, key, value, k_cache, v_cache, block_tables, seq_lens, scale, workspace,
                              partition_tokens=0, stream=None, flags=0):
    """The first phase of ``pa_decode_step`` (then ``pa_decode_merge``)."""
    nb, bs, hkv, d, b, hq, mb = _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens)
    _new_rows(key, value, q, hkv, d)
    need = pa_decode_workspace_size(b, hq, hkv, d, bs, mb, partition_tokens)
    ws, ws_bytes = _workspace(workspace, need, q.device)
    _check("pa_decode_partitions_step", lib.pa_decode_partitions_step(
        _ptr(out), _ptr(q), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(seq_lens), b, hq, hkv, d, bs, mb, nb, float(scale), _kv_dtype(k_cache), partition_tokens, flags,
        _ptr(ws), ws_bytes, _stream(stream)))


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, seq_lens, scale, partition_tokens=0,
                      stream=None, flags=0):
    """``pa_decode`` without a workspace: the split-KV partials go to the library's
    static per-GPU scratch (``NOALLOC_SCRATCH_BYTES``), so nothing is allocated.
    Calls that overlap in time on one GPU race on that scratch."""
    nb, bs, hkv, d, b, hq, mb = _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens)
    _check("pa_decode_noalloc", lib.pa_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens), b, hq,
        hkv, d, bs, mb, nb, float(scale), _kv_dtype(k_cache), partition_tokens, flags,
        _stream(stream)))
    return out


def pa_decode_multi(out, q, k_cache, v_cache, block_tables, seq_lens, scale, partition_tokens=0,
                    workspace=None, stream=None, flags=0):
    """Decode with several new queries per sequence (draft-token verification):
    ``q``/``out`` are ``[B, Q, Hq, D]``; query ``j`` of sequence ``b`` sits at position
    ``seq_lens[b] - Q + j`` and sees the keys up to it."""
    _need(k_cache, "k_cache", ndim=4)
    _need(v_cache, "v_cache", k_cache.dtype, 4)
    _need(q, "q", k_cache.dtype, 4)
    _need(out, "out", k_cache.dtype, 4)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    nb, bs, hkv, d = k_cache.shape
    b, nq, hq, dq = q.shape
    if v_cache.shape != k_cache.shape or out.shape != q.shape or dq != d:
        raise ValueError("q/out/cache shapes disagree")
    if block_tables.shape[0] != b or seq_lens.shape[0] != b:
        raise ValueError("block_tables and seq_lens need one row per sequence")
    mb = block_tables.shape[1]
    need = pa_decode_workspace_size(b * nq, hq, hkv, d, bs, mb, partition_tokens)
    ws, ws_bytes = _workspace(workspace, need, q.device)
    _check("pa_decode_multi", lib.pa_decode_multi(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens), b, nq,
        hq, hkv, d, bs, mb, nb, float(scale), _kv_dtype(k_cache), partition_tokens, flags, _ptr(ws),
        ws_bytes, _stream(stream)))
    return out


def pa_decode_partitions(out, q, k_cache, v_cache, block_tables, seq_lens, scale, workspace,
                         partition_tokens=0, stream=None, flags=0):
    nb, bs, hkv, d, b, hq, mb = _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens)
    need = pa_decode_workspace_size(b, hq, hkv, d, bs, mb, partition_tokens)
    ws, ws_bytes = _workspace(workspace, need, q.device)
    _check("pa_decode_partitions", lib.pa_decode_partitions(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens), b, hq,
        hkv, d, bs, mb, nb, float(scale), _kv_dtype(k_cache), partition_tokens, flags, _ptr(ws), ws_bytes,
        _stream(stream)))


def pa_decode_merge(out, seq_lens, num_kv_heads, max_blocks_per_seq, workspace,
                    partition_tokens=0, stream=None, block_size=BLOCK_SIZE):
    _need(out, "out", ndim=3)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    b, hq, d = out.shape
    need = pa_decode_workspace_size(b, hq, num_kv_heads, d, block_size, max_blocks_per_seq,
                                    partition_tokens)
    ws, ws_bytes = _workspace(workspace, need, out.device)
    _check("pa_decode_merge", lib.pa_decode_merge(
        _ptr(out), _ptr(seq_lens), b, hq, num_kv_heads, d, block_size, max_blocks_per_seq,
        _kv_dtype(out), partition_tokens, _ptr(ws), ws_bytes, _stream(stream)))


def pa_prefill_paged(out, q, k_cache, v_cache, block_tables, ctx_lens, query_start_loc, scale,
                     max_q_len, stream=None):
    """Causal chunked prefill of the packed rows ``q`` (``[T, Hq, D]``) into ``out``.
    ``max_q_len`` is a host-side upper bound of any sequence's row count."""
    _need(k_cache, "k_cache", ndim=4)
    _need(v_cache, "v_cache", k_cache.dtype, 4)
    _need(q, "q", k_cache.dtype, 3)
    _need(out, "out", k_cache.dtype, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(ctx_lens, "ctx_lens", torch.int32, 1)
    _need(query_start_loc, "query_start_loc", torch.int32, 1)
    nb, bs, hkv, d = k_cache.shape
    t, hq, dq = q.shape
    b = ctx_lens.shape[0]
    if v_cache.shape != k_cache.shape or out.shape != q.shape or dq != d:
        raise ValueError("q/out/cache shapes disagree")
    if block_tables.shape[0] != b or query_start_loc.shape[0] != b + 1:
        raise ValueError("block_tables / query_start_loc do not match ctx_lens")
    _check("pa_prefill_paged", lib.pa_prefill_paged(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(ctx_lens),
        _ptr(query_start_loc), b, t, int(max_q_len), hq, hkv, d, bs, block_tables.shape[1], nb,
        float(scale), _kv_dtype(k_cache), _stream(stream)))
    return out


# ------------------------------------------------------------- FP8 KV cache

def _fp8_pools(k_cache, v_cache, k_scales, v_scales):
    _need(k_cache, "k_cache", torch.uint8, 4)
    _need(v_cache, "v_cache", torch.uint8, 4)
    _need(k_scales, "k_scales", torch.float32, 3)
    _need(v_scales, "v_scales", torch.float32, 3)
    nb, bs, hkv, d = k_cache.shape
    if v_cache.shape != k_cache.shape or k_scales.shape != (nb, hkv, bs) or v_scales.shape != (nb, hkv, bs):
        raise ValueError("FP8 pools need codes [NB, 16, Hkv, D] and scales [NB, Hkv, 16]")
    return nb, bs, hkv, d


def pa_reshape_and_cache_fp8(key, value, k_cache, v_cache, k_scales, v_scales, slot_mapping,
                             stream=None):
    """Quantise ``key[t]``/``value[t]`` (``[N, Hkv, D]``, fp16 or bf16) to E4M3 with one
    float32 scale per (token, kv head) and store codes and scales at slot
    ``slot_mapping[t]``; negative slots are skipped."""
    nb, bs, hkv, d = _fp8_pools(k_cache, v_cache, k_scales, v_scales)
    _need(key, "key", None, 3)
    _need(value, "value", key.dtype, 3)
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    if key.shape != value.shape or tuple(key.shape[1:]) != (hkv, d):
        raise ValueError("key/value/cache shapes disagree")
    if slot_mapping.shape[0] != key.shape[0]:
        raise ValueError("slot_mapping needs one entry per token")
    _check("pa_reshape_and_cache_fp8", lib.pa_reshape_and_cache_fp8(
        _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
        _ptr(slot_mapping), key.shape[0], hkv, d, bs, nb, _kv_dtype(key), _stream(stream)))


def pa_copy_blocks_fp8(k_cache, v_cache, k_scales, v_scales, block_pairs, stream=None):
    """Copy whole blocks of an FP8 cache (codes and scales): ``block_pairs`` is int64
    ``[N, 2]`` of (src, dst) rows."""
    nb, bs, hkv, d = _fp8_pools(k_cache, v_cache, k_scales, v_scales)
    _need(block_pairs, "block_pairs", torch.int64, 2)
    if block_pairs.shape[1] != 2:
        raise ValueError("block_pairs is not [N, 2]")
    _check("pa_copy_blocks_fp8", lib.pa_copy_blocks_fp8(
        _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales), _ptr(block_pairs),
        block_pairs.shape[0], hkv, d, bs, nb, _stream(stream)))


def _decode_fp8_args(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens):
    nb, bs, hkv, d = _fp8_pools(k_cache, v_cache, k_scales, v_scales)
    _need(q, "q", None, 3)
    _need(out, "out", q.dtype, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    b, hq, dq = q.shape
    if out.shape != q.shape or dq != d:
        raise ValueError("q/out/cache shapes disagree")
    if block_tables.shape[0] != b or seq_lens.shape[0] != b:
        raise ValueError("block_tables and seq_lens need one row per sequence")
    return nb, bs, hkv, d, b, hq, block_tables.shape[1]


def pa_decode_fp8(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens, scale,
                  partition_tokens=0, workspace=None, stream=None, flags=0):
    """Paged decode over an FP8 cache into ``out`` (``[B, Hq, D]``, the type of ``q``);
    the other arguments as for ``pa_decode``."""
    nb, bs, hkv, d, b, hq, mb = _decode_fp8_args(out, q, k_cache, v_cache, k_scales, v_scales,
                                                 block_tables, seq_lens)
    need = pa_decode_workspace_size(b, hq, hkv, d, bs, mb, partition_tokens)
    ws, ws_bytes = _workspace(workspace, need, q.device)
    _check("pa_decode_fp8", lib.pa_decode_fp8(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
        _ptr(block_tables), _ptr(seq_lens), b, hq, hkv, d, bs, mb, nb, float(scale), _kv_dtype(q),
        partition_tokens, flags, _ptr(ws), ws_bytes, _stream(stream)))
    return out


def pa_decode_partitions_fp8(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                             scale, workspace, partition_tokens=0, stream=None, flags=0):
    nb, bs, hkv, d, b, hq, mb = _decode_fp8_args(out, q, k_cache, v_cache, k_scales, v_scales,
                                                 block_tables, seq_lens)
    need = pa_decode_workspace_size(b, hq, hkv, d, bs, mb, partition_tokens)
    ws, ws_bytes = _workspace(workspace, need, q.device)
    _check("pa_decode_partitions_fp8", lib.pa_decode_partitions_fp8(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
        _ptr(block_tables), _ptr(seq_lens), b, hq, hkv, d, bs, mb, nb, float(scale), _kv_dtype(q),
        partition_tokens, flags, _ptr(ws), ws_bytes, _stream(stream)))


def pa_prefill_paged_fp8(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, ctx_lens,
                         query_start_loc, scale, max_q_len, stream=None):
    """Causal chunked prefill of the packed rows ``q`` over an FP8 cache into ``out``;
    the other arguments as for ``pa_prefill_paged``."""
    nb, bs, hkv, d = _fp8_pools(k_cache, v_cache, k_scales, v_scales)
    _need(q, "q", None, 3)
    _need(out, "out", q.dtype, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(ctx_lens, "ctx_lens", torch.int32, 1)
    _need(query_start_loc, "query_start_loc", torch.int32, 1)
    t, hq, dq = q.shape
    b = ctx_lens.shape[0]
    if out.shape != q.shape or dq != d:
        raise ValueError("q/out/cache shapes disagree")
    if block_tables.shape[0] != b or query_start_loc.shape[0] != b + 1:
        raise ValueError("block_tables / query_start_loc do not match ctx_lens")
    _check("pa_prefill_paged_fp8", lib.pa_prefill_paged_fp8(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
        _ptr(block_tables), _ptr(ctx_lens), _ptr(query_start_loc), b, t, int(max_q_len), hq, hkv, d,
        bs, block_tables.shape[1], nb, float(scale), _kv_dtype(q), _stream(stream)))
    return out


def pa_debug_bounds(clear: bool = True, stream=None) -> int:
    """The bits the index checks of a debug build (libpa_debug.so, loaded with
    PA_DEBUG_BOUNDS=1) set since the last clear; waits for the stream.  Raises
    PagedKVError (unsupported) with the normal library."""
    word = _u32(0)
    _check("pa_debug_bounds", lib.pa_debug_bounds(ctypes.byref(word), 1 if clear else 0, _stream(stream)))
    return int(word.value)
