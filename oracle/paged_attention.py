"""Float64 CPU oracle for the paged KV-cache attention hot path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product package.

What it computes, and where the pages fix it
--------------------------------------------
* Paging only changes *where* K/V live, never what attention computes.  The
  KV cache is cut into fixed-size blocks held in one global pool, and each
  sequence keeps a block table from logical to physical blocks
  ["vLLM-Ascend 原理", §2.1 "PagedAttention 分页 KV 缓存"; "vLLM学习整理",
  §三 "PagedAttention"].  So every attention function below first reads the
  sequence's tokens in logical order through the table, then applies the
  textbook definition.
* Token ``p`` of a sequence is in physical block ``table[p // block_size]`` at
  offset ``p % block_size``; this is how ``read_kv`` in the ``PagedKVCache``
  sketch addresses the pool ["vLLM 在 CANN 上的推理优化", section
  "vLLM 的 PagedAttention 数据结构"].
* Causal self-attention: the query at position ``i`` is dotted with the keys
  at positions ``0..i``, softmax, then a weighted sum of the values; under GQA
  several q heads share one k/v head ["vLLM-Ascend 原理", §2.3 "Prefill",
  step 3].  Decode is the same with a single new query at the last position,
  reading the whole prefix through the block table ["vLLM-Ascend 原理", §2.4
  "Decode", step 3].
* The cache write puts each new token's k and v into its slot of a physical
  block ["vLLM-Ascend 原理", §2.3 step 3 and §2.4 step 3].
* Chunked prefill: a later chunk attends to the KV that earlier chunks already
  wrote to the cache ["vLLM-Ascend 原理", §2.4, closing paragraphs on chunked
  prefill].
* KV bytes per token = 2 x layers x kv_heads x head_dim x dtype_size
  ["vLLM-Ascend 原理", §2.1, the KV size formula].
* Online softmax merging block by block is an exact rewrite of softmax
  ["vLLM-Ascend 原理", §四 "ATB 算子"; "vLLM 在 CANN 上的推理优化", section
  "CANN 上的 PagedAttention 算子"].  ``ref_partition_state`` and
  ``ref_merge_partitions`` state that algebra plainly so it can be pinned.

Readings taken where the pages are silent (each also listed in the design
notes): K and V are separate ``[num_blocks, block_size, kv_heads, head_dim]``
tensors; a negative slot means "do not write"; ``seq_lens`` counts the current
token (the cache write happens before decode attention); ``ctx_lens`` counts
tokens cached before the chunk; q head ``h`` reads kv head ``h // G``; a
sequence of length 0 yields zeros; the scale is the float32 value the kernel
receives.

Storage is passed as raw 16-bit patterns (``numpy.uint16``) plus a dtype
name, ``"f16"`` or ``"bf16"``; both widen to float64 exactly.
"""

from __future__ import annotations

import numpy as np

DTYPES = ("f16", "bf16")


def bits_to_float64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen fp16 / bf16 bit patterns to float64 (exact for every value)."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError(f"expected uint16 bit patterns, got {bits.dtype}")
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        # a bf16 value is the top half of the float32 with the same bits
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def kernel_scale(scale: float) -> float:
    """The softmax scale as the kernel receives it: rounded to float32."""
    return float(np.float32(scale))


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """K and V bytes one token occupies across all layers.

    ["vLLM-Ascend 原理", §2.1]: 2 (K and V) x layers x kv_heads x head_dim x
    dtype size.
    """
    return 2 * layers * kv_heads * head_dim * dtype_bytes


def ref_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping):
    """Scatter each new token's k and v into its cache slot (bit copy).

    ["vLLM-Ascend 原理", §2.3 step 3 / §2.4 step 3]: new k, v are written into
    physical blocks through the block table, a block holding ``block_size``
    tokens.  A slot ``s`` names block ``s // block_size`` and offset
    ``s % block_size``.  Negative slots are padding rows and are skipped.
    Slots must be distinct and inside the pool.

    Returns new ``(k_cache, v_cache)`` arrays; the inputs are not modified.
    """
    key = np.asarray(key)
    value = np.asarray(value)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
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
        kc[block, offset] = key[t]
        vc[block, offset] = value[t]
    return kc, vc


def ref_copy_blocks(k_cache, v_cache, block_pairs):
    """Copy whole physical blocks, K and V: block ``dst`` becomes a copy of block
    ``src`` for every ``(src, dst)`` pair.

    This is the block copy behind copy-on-write: sequences that share a prefix
    point at the same physical blocks until one of them writes, and then forks
    onto a copy ["vLLM-Ascend 原理", §2.1, prefix sharing with copy-on-write];
    the same copy moves blocks for swapping ["vLLM学习整理", §三 "Preemption"].
    Pairs with a negative entry are skipped.  Destinations must be distinct and
    no destination may also be a source, so the order of the pairs does not
    matter.  Returns new ``(k_cache, v_cache)``.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    num_blocks = kc.shape[0]
    pairs = [(int(a), int(b)) for a, b in np.asarray(block_pairs).reshape(-1, 2)]
    live = [(a, b) for a, b in pairs if a >= 0 and b >= 0]
    dsts = [b for _, b in live]
    if len(set(dsts)) != len(dsts):
        raise ValueError("a destination block appears twice")
    for a, b in live:
        if a >= num_blocks or b >= num_blocks:
            raise IndexError(f"block pair ({a}, {b}) outside a pool of {num_blocks}")
    if any(b in {a for a, _ in live} and (b, b) not in live for b in dsts):
        raise ValueError("a destination block is also a source")
    for a, b in live:
        kc[b] = k_cache[a]
        vc[b] = v_cache[a]
    return kc, vc


def gather_tokens(cache: np.ndarray, table_row: np.ndarray, n: int) -> np.ndarray:
    """The first ``n`` tokens of one sequence, in logical order.

    ["vLLM 在 CANN 上的推理优化", ``read_kv``]: logical token ``p`` is at offset
    ``p % block_size`` of physical block ``table_row[p // block_size]``.
    Returns ``[n, kv_heads, head_dim]`` with the cache's element type.
    """
    block_size = cache.shape[1]
    p = np.arange(n)
    physical = np.asarray(table_row)[p // block_size]
    return cache[physical, p % block_size]


def ref_contiguous_attention(q, k, v, scale, q_pos):
    """Textbook causal softmax attention with GQA, in float64.

    ``q``: ``[Lq, Hq, D]``; ``k``, ``v``: ``[Lk, Hkv, D]`` (float64, contiguous
    logical order).  Row ``i`` sits at logical position ``q_pos[i]`` and sees
    keys ``0..q_pos[i]`` inclusive ["vLLM-Ascend 原理", §2.3 step 3].  With
    ``G = Hq // Hkv``, q head ``h`` reads kv head ``h // G``.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    q_pos = np.asarray(q_pos)
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    if hq % hkv:
        raise ValueError("q heads must be a multiple of kv heads")
    if lq and q_pos.max() >= lk:
        raise ValueError("a query position reaches past the keys")
    group = hq // hkv
    scale = kernel_scale(scale)
    out = np.zeros((lq, hq, d))
    visible = np.arange(lk)[None, :] <= q_pos[:, None]          # [Lq, Lk]
    for h in range(hq):
        g = h // group
        s = scale * (q[:, h, :] @ k[:, g, :].T)                  # [Lq, Lk]
        s = np.where(visible, s, -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ v[:, g, :]
    return out


def ref_decode_one(q_b, k_cache, v_cache, table_row, n, scale, dtype):
    """Decode attention for one sequence: its query ``q_b`` (``[Hq, D]`` bits)
    attends to all ``n`` cached tokens, read through the block table
    ["vLLM-Ascend 原理", §2.4 step 3].  ``n == 0`` gives zeros."""
    hq, d = q_b.shape
    if n == 0:
        return np.zeros((hq, d))
    k = bits_to_float64(gather_tokens(k_cache, table_row, n), dtype)
    v = bits_to_float64(gather_tokens(v_cache, table_row, n), dtype)
    q = bits_to_float64(q_b, dtype)[None]
    return ref_contiguous_attention(q, k, v, scale, np.array([n - 1]))[0]


def ref_decode(q, k_cache, v_cache, block_tables, seq_lens, scale, dtype):
    """Paged decode for a batch: ``q`` ``[B, Hq, D]`` bits -> float64
    ``[B, Hq, D]``.  ``seq_lens[b]`` counts the current token, whose k/v the
    cache write has already stored."""
    out = np.zeros(q.shape, np.float64)
    for b in range(q.shape[0]):
        out[b] = ref_decode_one(q[b], k_cache, v_cache, block_tables[b],
                                int(seq_lens[b]), scale, dtype)
    return out


def ref_decode_multi(q, k_cache, v_cache, block_tables, seq_lens, scale, dtype):
    """Decode with several new queries per sequence, as speculative decoding
    verifies its draft tokens: the k proposed tokens plus the last accepted one
    are scored in one pass over the cache ["vLLM-Ascend 原理", §四, the
    speculative-decoding paragraphs: the target model checks all k draft
    tokens at once, like a small prefill].

    ``q``: ``[B, Q, Hq, D]`` bits.  ``seq_lens[b] = n`` counts every cached token
    including the Q new ones (already written); query ``j`` sits at position
    ``n - Q + j`` and sees keys ``0 .. n - Q + j`` (causal among the new
    tokens).  A query whose position is negative (``n < Q - j``) gives zeros.
    Returns float64 ``[B, Q, Hq, D]``.
    """
    bsz, nq, hq, d = q.shape
    out = np.zeros(q.shape, np.float64)
    for b in range(bsz):
        n = int(seq_lens[b])
        pos = n - nq + np.arange(nq)
        live = np.flatnonzero(pos >= 0)
        if live.size == 0:
            continue
        k = bits_to_float64(gather_tokens(k_cache, block_tables[b], n), dtype)
        v = bits_to_float64(gather_tokens(v_cache, block_tables[b], n), dtype)
        qb = bits_to_float64(q[b, live], dtype)
        out[b, live] = ref_contiguous_attention(qb, k, v, scale, pos[live])
    return out


def ref_prefill_rows(q, k_cache, v_cache, table_row, ctx_len, row_start, rows,
                     scale, dtype):
    """Chunked-prefill attention for some rows of one sequence.

    The sequence's new rows are ``q[row_start + i]`` at logical positions
    ``ctx_len + i``; ``rows`` picks which ``i`` to compute.  Keys ``0..ctx_len+i``
    are read through the table: the cached context plus this chunk's own
    tokens, already written ["vLLM-Ascend 原理", §2.3 step 3 and §2.4 on
    chunked prefill].  Returns float64 ``[len(rows), Hq, D]``.
    """
    rows = np.asarray(rows, np.int64)
    if rows.size == 0:
        return np.zeros((0,) + q.shape[1:])
    n = ctx_len + int(rows.max()) + 1
    k = bits_to_float64(gather_tokens(k_cache, table_row, n), dtype)
    v = bits_to_float64(gather_tokens(v_cache, table_row, n), dtype)
    qr = bits_to_float64(q[row_start + rows], dtype)
    return ref_contiguous_attention(qr, k, v, scale, ctx_len + rows)


def ref_prefill_paged(q, k_cache, v_cache, block_tables, ctx_lens, query_start_loc,
                      scale, dtype):
    """Chunked prefill for a batch of packed query rows ``q`` ``[T, Hq, D]``.

    Sequence ``b`` owns rows ``query_start_loc[b] .. query_start_loc[b+1]-1``.
    Returns float64 ``[T, Hq, D]``; rows owned by no sequence stay zero.
    """
    out = np.zeros(q.shape, np.float64)
    qsl = np.asarray(query_start_loc)
    for b in range(len(ctx_lens)):
        start, end = int(qsl[b]), int(qsl[b + 1])
        if end > start:
            out[start:end] = ref_prefill_rows(q, k_cache, v_cache, block_tables[b],
                                              int(ctx_lens[b]), start,
                                              np.arange(end - start), scale, dtype)
    return out


def ref_partition_state(q, k, v, scale, start, end):
    """Softmax state of one query over keys ``start..end-1`` (float64).

    ``q``: ``[Hq, D]``; ``k``, ``v``: ``[Lk, Hkv, D]``.  Returns ``(m, l, acc)``
    with ``m[h]`` the largest score, ``l[h] = sum exp(s - m)`` and
    ``acc[h] = sum exp(s - m) * v``: the running statistics an online softmax
    keeps while it walks the blocks ["vLLM-Ascend 原理", §四 "ATB 算子"].
    """
    q = np.asarray(q, np.float64)
    hq, d = q.shape
    group = hq // k.shape[1]
    scale = kernel_scale(scale)
    m = np.empty(hq)
    l = np.empty(hq)
    acc = np.empty((hq, d))
    for h in range(hq):
        kg = np.asarray(k[start:end, h // group], np.float64)
        vg = np.asarray(v[start:end, h // group], np.float64)
        s = scale * (kg @ q[h])
        m[h] = s.max()
        e = np.exp(s - m[h])
        l[h] = e.sum()
        acc[h] = e @ vg
    return m, l, acc


def ref_merge_partitions(ms, ls, accs):
    """Combine softmax states of disjoint key ranges into the attention output.

    With ``M = max_p m_p``: ``out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p``.
    ``ms``, ``ls``: ``[P, Hq]``; ``accs``: ``[P, Hq, D]``.
    """
    ms = np.asarray(ms, np.float64)
    big_m = ms.max(axis=0)
    w = np.exp(ms - big_m)                                     # [P, Hq]
    num = (w[:, :, None] * np.asarray(accs, np.float64)).sum(axis=0)
    den = (w * np.asarray(ls, np.float64)).sum(axis=0)
    return num / den[:, None]
