"""Float64 CPU oracle for an FP8 (E4M3) paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product package.

What the pages fix ["vLLM-Ascend 原理", §四, the paragraph on KV-cache
quantisation]: each layer's per-head k and v are stored in 8 bits instead of
16, which halves the cache; the values are quantised when the decode step
writes them, and after the block-table lookup they are dequantised before the
attention arithmetic, inside the paged attention operator.

Readings taken where the pages are silent (each also listed in the design
notes):

* The 8-bit format is the OCP 8-bit floating-point E4M3 encoding: sign bit,
  4 exponent bits with bias 7, 3 mantissa bits, subnormals at exponent 0, no
  infinities, S.1111.111 the only NaN, largest finite magnitude 448.
* One float32 scale per (token, kv head), shared by the head_dim elements of
  that row: ``s = amax / 448`` in float32 (``amax`` = largest magnitude in the
  row), and ``s = 1`` for an all-zero row.
* Each element is stored as ``e4m3(x / s)``, the quotient taken in float32
  (IEEE, correctly rounded) and converted with round-to-nearest-even, ties to
  the even code, magnitudes above 448 clamped to 448 (they only arise from
  the float32 rounding of the quotient).
* Dequantised value = ``decode(code) * s``, exact in float64; attention then
  follows the unquantised oracle on those values, q and out keeping the
  16-bit type.
* The scales live in their own pools ``[num_blocks, kv_heads, block_size]``
  (float32), beside the code pools ``[num_blocks, block_size, kv_heads,
  head_dim]`` (uint8).
"""

from __future__ import annotations

import numpy as np

from .paged_attention import (
    bits_to_float64,
    gather_tokens,
    ref_contiguous_attention,
)

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6       # smallest normal magnitude is 2**-6
_SUBNORMAL_STEP_EXP = -9   # spacing of the subnormals: 2**-9


def e4m3_to_float64(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8), from the format's definition.

    Exponent field ``e`` and mantissa ``m``: ``e == 0`` is subnormal,
    ``m/8 * 2**-6``; otherwise ``(1 + m/8) * 2**(e - 7)``; ``e == 15, m == 7``
    is NaN.  The sign bit negates.
    """
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError(f"expected uint8 codes, got {c.dtype}")
    c = c.astype(np.int64)
    sign = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m / 8.0, _MIN_NORMAL_EXP)
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def float_to_e4m3(x) -> np.ndarray:
    """Nearest E4M3 code to each value (ties to the even code), magnitudes
    clamped to 448 first.  ``x`` holds float64 values; NaN is rejected."""
    x = np.asarray(x, np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no saturating E4M3 encoding here")
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.minimum(np.abs(x), E4M3_MAX)
    # spacing of the codes around a: 2**(floor(log2 a) - 3) among the normals,
    # 2**-9 below the smallest normal
    _, e = np.frexp(a)                       # a = f * 2**e, 0.5 <= f < 1
    step = np.where(a < 2.0 ** _MIN_NORMAL_EXP, _SUBNORMAL_STEP_EXP, e - 1 - 3)
    steps = np.rint(np.ldexp(a, -step))      # round half to even on the step count
    v = np.ldexp(steps, step)                # the rounded magnitude, exact
    # encode the rounded magnitude
    _, ev = np.frexp(v)
    unbiased = ev - 1
    is_sub = v < 2.0 ** _MIN_NORMAL_EXP
    exp_field = np.where(is_sub, 0, unbiased + 7)
    mant = np.where(is_sub, np.ldexp(v, -_SUBNORMAL_STEP_EXP),
                    np.ldexp(v, -unbiased) * 8.0 - 8.0)
    code = sign | (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    return code.astype(np.uint8)


def quantize_e4m3_rows(x_bits, dtype: str):
    """Quantise rows of 16-bit values (last axis = one (token, head) row).

    Returns ``(codes uint8, same shape; scales float32, shape[:-1])`` following
    the per-row scale reading in the module docstring.
    """
    x = bits_to_float64(x_bits, dtype).astype(np.float32)   # exact
    if not np.isfinite(x).all():
        raise ValueError("only finite values are quantised")
    amax = np.abs(x).max(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        y = (x / scale[..., None]).astype(np.float32)       # float32 quotient
    return float_to_e4m3(y.astype(np.float64)), scale


def dequantize_e4m3_rows(codes, scales) -> np.ndarray:
    """``decode(code) * scale`` in float64 (exact); ``scales`` has one entry per
    row of ``codes``."""
    return e4m3_to_float64(codes) * np.asarray(scales, np.float32).astype(np.float64)[..., None]


def ref_reshape_and_cache_fp8(key, value, k_cache, v_cache, k_scales, v_scales,
                              slot_mapping, dtype: str):
    """Quantise each new token's k and v per kv head and scatter the codes and
    scales into the token's slot ["vLLM-Ascend 原理", §四: quantised as the
    decode step writes them; §2.3 step 3 / §2.4 step 3 for the slot].

    Slot ``s`` is block ``s // block_size``, offset ``s % block_size``; its codes
    go to ``cache[block, offset]`` and its per-head scales to
    ``scales[block, :, offset]``.  Negative slots are skipped; slots must be
    distinct and inside the pool.  Returns new ``(k_cache, v_cache, k_scales,
    v_scales)``.
    """
    kq, ks = quantize_e4m3_rows(key, dtype)
    vq, vs = quantize_e4m3_rows(value, dtype)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    ksc = np.array(k_scales, copy=True)
    vsc = np.array(v_scales, copy=True)
    num_blocks, block_size = kc.shape[0], kc.shape[1]
    seen = set()
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        if s >= num_blocks * block_size:
            raise IndexError(f"slot {s} outside a pool of {num_blocks} x {block_size}")
        if s in seen:
            raise ValueError(f"slot {s} written twice")
        seen.add(s)
        block, offset = divmod(s, block_size)
        kc[block, offset] = kq[t]
        vc[block, offset] = vq[t]
        ksc[block, :, offset] = ks[t]
        vsc[block, :, offset] = vs[t]
    return kc, vc, ksc, vsc


def gather_scales(scales: np.ndarray, table_row: np.ndarray, n: int) -> np.ndarray:
    """Per-head scales of the first ``n`` tokens of a sequence, logical order:
    token ``p`` is at offset ``p % block_size`` of physical block
    ``table_row[p // block_size]`` ["vLLM 在 CANN 上的推理优化", ``read_kv``].
    Returns ``[n, kv_heads]`` float32."""
    block_size = scales.shape[2]
    p = np.arange(n)
    physical = np.asarray(table_row)[p // block_size]
    return scales[physical, :, p % block_size]


def _dequantized_tokens(codes, scales, table_row, n):
    return dequantize_e4m3_rows(gather_tokens(codes, table_row, n),
                                gather_scales(scales, table_row, n))


def ref_decode_fp8(q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                   scale, dtype: str):
    """Paged decode over an E4M3 cache: K/V are read through the block table,
    dequantised, then attended to as in the unquantised oracle
    ["vLLM-Ascend 原理", §四 and §2.4 step 3].  ``q`` holds 16-bit patterns of
    ``dtype``; returns float64 ``[B, Hq, D]``; a length-0 sequence gives zeros."""
    out = np.zeros(q.shape, np.float64)
    for b in range(q.shape[0]):
        n = int(seq_lens[b])
        if n == 0:
            continue
        k = _dequantized_tokens(k_cache, k_scales, block_tables[b], n)
        v = _dequantized_tokens(v_cache, v_scales, block_tables[b], n)
        qb = bits_to_float64(q[b], dtype)[None]
        out[b] = ref_contiguous_attention(qb, k, v, scale, np.array([n - 1]))[0]
    return out


def ref_prefill_rows_fp8(q, k_cache, v_cache, k_scales, v_scales, table_row, ctx_len,
                         row_start, rows, scale, dtype: str):
    """Chunked-prefill rows of one sequence over an E4M3 cache (see
    ``ref_prefill_rows`` of the unquantised oracle for the positions)."""
    rows = np.asarray(rows, np.int64)
    if rows.size == 0:
        return np.zeros((0,) + q.shape[1:])
    n = ctx_len + int(rows.max()) + 1
    k = _dequantized_tokens(k_cache, k_scales, table_row, n)
    v = _dequantized_tokens(v_cache, v_scales, table_row, n)
    qr = bits_to_float64(q[row_start + rows], dtype)
    return ref_contiguous_attention(qr, k, v, scale, ctx_len + rows)


def ref_prefill_paged_fp8(q, k_cache, v_cache, k_scales, v_scales, block_tables,
                          ctx_lens, query_start_loc, scale, dtype: str):
    """Chunked prefill for packed rows ``q`` ``[T, Hq, D]`` over an E4M3 cache;
    rows owned by no sequence stay zero."""
    out = np.zeros(q.shape, np.float64)
    qsl = np.asarray(query_start_loc)
    for b in range(len(ctx_lens)):
        start, end = int(qsl[b]), int(qsl[b + 1])
        if end > start:
            out[start:end] = ref_prefill_rows_fp8(q, k_cache, v_cache, k_scales, v_scales,
                                                  block_tables[b], int(ctx_lens[b]), start,
                                                  np.arange(end - start), scale, dtype)
    return out
