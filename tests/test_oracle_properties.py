"""Property tests of the oracle (Hypothesis, CPU): random shapes, lengths and
block placements, each checked against something other than the oracle.

* Paged decode and chunked prefill against torch's float64 scaled-dot-product
  attention on K/V that the test lays out itself: the test writes each
  sequence's logical K/V into a randomly permuted pool with its own loop, so
  the oracle's gather through the table, its GQA head mapping (q head h reads
  kv head h // G, expanded here with repeat_interleave) and its causal
  visibility are all pinned by an independent routine.
* The split-KV merge of random disjoint key ranges against the unsplit result
  (the algebra of the online softmax is exact up to rounding).
* The cache write against a brute-force loop over random slot mappings with
  padding slots (-1), bit for bit.
* The E4M3 row quantiser against the rounding bound of the format: every
  decoded code lies within half a code spacing of the float32 quotient.

Lengths are drawn with the edges of a paged layout (0, 1, block - 1, block,
block + 1, multiples) as well as from a range; the draws are derandomised.
"""

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

PROPS = settings(max_examples=40, deadline=None, derandomize=True, database=None,
                 suppress_health_check=[HealthCheck.too_slow])
LENS = st.one_of(st.sampled_from([0, 1, 15, 16, 17, 31, 32, 33, 48, 64]), st.integers(0, 90))


def _f16_bits(x):
    return np.asarray(x, np.float16).view(np.uint16)


def _pool_from_sequences(seqs, block_size, spare, rng):
    """Scatter each sequence's logical rows [n, H, D] (float16 values) into a
    pool of randomly permuted blocks; returns (pool bits, tables)."""
    h, d = seqs[0].shape[1:] if seqs else (1, 1)
    need = [(len(s) + block_size - 1) // block_size for s in seqs]
    nb = sum(need) + spare
    perm = rng.permutation(max(nb, 1))
    pool = np.full((max(nb, 1), block_size, h, d), 0x7E00, np.uint16)   # NaN in unused slots
    mb = max(need + [1])
    tables = np.full((len(seqs), mb), -1, np.int32)
    cur = 0
    for b, s in enumerate(seqs):
        for j in range(need[b]):
            tables[b, j] = perm[cur]
            cur += 1
        for p in range(len(s)):
            pool[tables[b, p // block_size], p % block_size] = _f16_bits(s[p])
    return pool, tables


def _sdpa(q, k, v, scale, visible):
    """torch float64 attention; q [Lq, Hq, D], k/v [Lk, Hkv, D], visible [Lq, Lk]."""
    hq, hkv = q.shape[1], k.shape[1]
    kq = torch.from_numpy(k).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)
    vq = torch.from_numpy(v).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)
    qt = torch.from_numpy(q).permute(1, 0, 2)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kq.contiguous(), vq.contiguous(), attn_mask=torch.from_numpy(visible), scale=scale)
    return out.permute(1, 0, 2).numpy()


@st.composite
def shapes(draw):
    hkv = draw(st.sampled_from([1, 2]))
    g = draw(st.sampled_from([1, 2, 3]))
    d = draw(st.sampled_from([8, 16]))
    bs = draw(st.sampled_from([16, 32]))
    return hkv, g, d, bs


@PROPS
@given(shapes(), st.lists(LENS, min_size=1, max_size=4), st.integers(0, 4), st.integers(0, 2 ** 31))
def test_paged_decode_equals_sdpa(shape, lens, spare, seed):
    hkv, g, d, bs = shape
    rng = np.random.default_rng(seed)
    seqs = [rng.standard_normal((n, hkv, d)).astype(np.float16) for n in lens]
    vals = [rng.standard_normal((n, hkv, d)).astype(np.float16) for n in lens]
    kpool, tables = _pool_from_sequences(seqs, bs, spare, np.random.default_rng(seed + 1))
    vpool, tables_v = _pool_from_sequences(vals, bs, spare, np.random.default_rng(seed + 1))
    assert (tables == tables_v).all()
    q = rng.standard_normal((len(lens), hkv * g, d)).astype(np.float16)
    scale = 0.3
    got = oracle.ref_decode(_f16_bits(q), kpool, vpool, tables, np.array(lens), scale, "f16")
    for b, n in enumerate(lens):
        if n == 0:
            assert (got[b] == 0).all()
            continue
        want = _sdpa(q[b:b + 1].astype(np.float64), seqs[b].astype(np.float64),
                     vals[b].astype(np.float64), float(np.float32(scale)), np.ones((1, n), bool))
        np.testing.assert_allclose(got[b], want[0], rtol=0, atol=1e-12)


@PROPS
@given(shapes(), st.lists(st.tuples(LENS, st.integers(0, 40)), min_size=1, max_size=3),
       st.integers(0, 2 ** 31))
def test_chunked_prefill_equals_sdpa(shape, ctx_and_len, seed):
    hkv, g, d, bs = shape
    rng = np.random.default_rng(seed)
    totals = [c + l for c, l in ctx_and_len]
    seqs = [rng.standard_normal((n, hkv, d)).astype(np.float16) for n in totals]
    vals = [rng.standard_normal((n, hkv, d)).astype(np.float16) for n in totals]
    kpool, tables = _pool_from_sequences(seqs, bs, 2, np.random.default_rng(seed + 1))
    vpool, _ = _pool_from_sequences(vals, bs, 2, np.random.default_rng(seed + 1))
    q_lens = np.array([l for _, l in ctx_and_len])
    qsl = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = rng.standard_normal((int(qsl[-1]), hkv * g, d)).astype(np.float16)
    scale = 0.25
    got = oracle.ref_prefill_paged(_f16_bits(q), kpool, vpool, tables,
                                   np.array([c for c, _ in ctx_and_len]), qsl, scale, "f16")
    for b, (ctx, l) in enumerate(ctx_and_len):
        if l == 0:
            continue
        visible = np.arange(ctx + l)[None, :] <= (ctx + np.arange(l))[:, None]
        want = _sdpa(q[qsl[b]:qsl[b + 1]].astype(np.float64), seqs[b].astype(np.float64),
                     vals[b].astype(np.float64), float(np.float32(scale)), visible)
        np.testing.assert_allclose(got[qsl[b]:qsl[b + 1]], want, rtol=0, atol=1e-12)


@PROPS
@given(st.integers(1, 200), st.lists(st.floats(0.0, 1.0), min_size=1, max_size=6),
       st.sampled_from([1, 2, 4]), st.integers(0, 2 ** 31))
def test_split_merge_equals_unsplit(n, cuts, group, seed):
    rng = np.random.default_rng(seed)
    d, hkv = 8, 2
    k = rng.standard_normal((n, hkv, d)) * 3
    v = rng.standard_normal((n, hkv, d))
    q = rng.standard_normal((hkv * group, d))
    edges = sorted({0, n, *[int(c * n) for c in cuts]})
    parts = [(a, b) for a, b in zip(edges, edges[1:]) if b > a]
    states = [oracle.ref_partition_state(q, k, v, 0.5, a, b) for a, b in parts]
    merged = oracle.ref_merge_partitions([s[0] for s in states], [s[1] for s in states],
                                         [s[2] for s in states])
    want = _sdpa(q[None], k, v, float(np.float32(0.5)), np.ones((1, n), bool))[0]
    np.testing.assert_allclose(merged, want, rtol=0, atol=1e-12)


@PROPS
@given(st.integers(1, 6), st.integers(1, 40), st.integers(0, 2 ** 31))
def test_cache_write_brute_force(num_blocks, num_tokens, seed):
    rng = np.random.default_rng(seed)
    bs, h, d = 16, 2, 4
    slots_avail = num_blocks * bs
    n = min(num_tokens, slots_avail)
    slots = rng.choice(slots_avail, size=n, replace=False).astype(np.int64)
    slots[rng.random(n) < 0.25] = -1                       # padding rows
    key = rng.integers(0, 2 ** 16, (n, h, d), dtype=np.uint16)
    value = rng.integers(0, 2 ** 16, (n, h, d), dtype=np.uint16)
    k0 = rng.integers(0, 2 ** 16, (num_blocks, bs, h, d), dtype=np.uint16)
    v0 = rng.integers(0, 2 ** 16, (num_blocks, bs, h, d), dtype=np.uint16)
    kc, vc = oracle.ref_reshape_and_cache(key, value, k0, v0, slots)
    want_k, want_v = k0.copy(), v0.copy()
    for t in range(n):
        s = int(slots[t])
        if s >= 0:
            want_k[s // bs, s % bs] = key[t]
            want_v[s // bs, s % bs] = value[t]
    np.testing.assert_array_equal(kc, want_k)
    np.testing.assert_array_equal(vc, want_v)


@PROPS
@given(st.integers(1, 8), st.integers(-14, 8), st.integers(0, 2 ** 31), st.sampled_from(["f16", "bf16"]))
def test_e4m3_rows_within_half_spacing(rows, exp, seed, dtype):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, 32)) * 2.0 ** exp
    x[rng.random((rows, 32)) < 0.1] = 0.0
    bits = (_f16_bits(x) if dtype == "f16"
            else (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    xs = oracle.bits_to_float64(bits, dtype)
    codes, scales = oracle.quantize_e4m3_rows(bits, dtype)
    dec = oracle.e4m3_to_float64(codes)
    assert np.isfinite(dec).all() and (np.abs(dec) <= 448).all()
    for r in range(rows):
        amax = np.abs(xs[r]).max()
        s = np.float32(scales[r])
        assert s == (np.float32(amax) / np.float32(448) if amax > 0 else np.float32(1))
        y = (xs[r].astype(np.float32) / s).astype(np.float64)           # the float32 quotient
        a = np.minimum(np.abs(y), 448.0)
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
        half = np.where(a < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))     # half a code spacing
        assert (np.abs(dec[r] - np.sign(y) * a) <= half).all()
