"""Checks that pin the float64 oracle to facts fixed outside itself.

Each ``pin_*`` function takes the oracle module and raises ``AssertionError``
when the oracle disagrees with a value the pages print, a closed form, a
library routine (torch's scaled-dot-product attention in float64), brute force
on a tiny input, or an invariant of the method.  ``test_oracle_pins.py`` runs
them on the real oracle; ``test_oracle_mutants.py`` plants mistakes in the
oracle and checks that some pin catches each one.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from workloads import make_decode_case, make_prefill_case, normal_bits, NAN_BITS

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand64(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa64(q, k, v, scale, q_pos):
    """torch's attention in float64 on the CPU, with an explicit causal mask.
    q [Lq, Hq, D], k/v [Lk, Hkv, D] -> [Lq, Hq, D]."""
    lk = k.shape[0]
    mask = torch.from_numpy(np.arange(lk)[None, :] <= np.asarray(q_pos)[:, None])
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=float(np.float32(scale)),
        enable_gqa=qt.shape[1] != kt.shape[1])
    return out[0].numpy().transpose(1, 0, 2)


# ---------------------------------------------------------------- page values

def pin_kv_bytes_golden(o):
    g = _golden("kv_bytes_llama2_7b.json")
    per_tok = o.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["dtype_bytes"])
    assert per_tok == g["bytes_per_token"]
    assert per_tok * g["sequence_tokens"] == g["sequence_bytes"]
    # GQA shrinks it by the group factor: 8 kv heads instead of 32
    assert o.kv_bytes_per_token(32, 8, 128, 2) * 4 == g["bytes_per_token"]


def pin_read_kv_addressing_golden(o):
    g = _golden("read_kv_addressing.json")
    bs = g["block_size"]
    table = np.array(g["block_table"], np.int32)
    nblocks = 8
    # every slot stores its own slot number (a 16-bit pattern)
    pool = np.arange(nblocks * bs, dtype=np.uint16).reshape(nblocks, bs, 1, 1)
    got = o.gather_tokens(pool, table, g["num_tokens"])[:, 0, 0]
    assert math.ceil(g["num_tokens"] / bs) == g["blocks_needed"]
    for lk in g["lookups"]:
        assert int(got[lk["token"]]) == lk["slot"]
        assert lk["slot"] == lk["physical_block"] * bs + lk["offset"]
    # the cache write puts a token at the same place
    empty = np.zeros((nblocks, bs, 1, 1), np.uint16)
    slots = np.array([lk["slot"] for lk in g["lookups"]], np.int64)
    key = (np.arange(len(slots), dtype=np.uint16) + 1).reshape(-1, 1, 1)
    kc, vc = o.ref_reshape_and_cache(key, key, empty, empty, slots)
    for i, lk in enumerate(g["lookups"]):
        assert int(kc[lk["physical_block"], lk["offset"], 0, 0]) == i + 1
        assert int(vc[lk["physical_block"], lk["offset"], 0, 0]) == i + 1
    assert int(np.count_nonzero(kc)) == len(slots)


def pin_two_keys_golden(o):
    g = _golden("softmax_two_keys.json")
    q = np.array(g["q"])[None, None, :]
    k = np.array(g["keys"])[:, None, :]
    v = np.array(g["values"])[:, None, :]
    out = o.ref_contiguous_attention(q, k, v, g["scale"], np.array([1]))[0, 0]
    np.testing.assert_allclose(out, g["expected_out"], rtol=0, atol=1e-14)


def pin_bits_widening(o):
    f16 = np.array([0x3C00, 0xC000, 0x0001, 0x7BFF, 0x3555], np.uint16)
    np.testing.assert_array_equal(o.bits_to_float64(f16, "f16"),
                                  [1.0, -2.0, 2.0 ** -24, 65504.0, 0.333251953125])
    bf16 = np.array([0x3F80, 0xC040, 0x0001, 0x4049, 0x3EAB], np.uint16)
    np.testing.assert_array_equal(o.bits_to_float64(bf16, "bf16"),
                                  [1.0, -3.0, 2.0 ** -133, 3.140625, 0.333984375])
    assert np.isnan(o.bits_to_float64(np.array([NAN_BITS["f16"]]), "f16")[0])
    assert np.isnan(o.bits_to_float64(np.array([NAN_BITS["bf16"]]), "bf16")[0])


# --------------------------------------------------------------- closed forms

def pin_single_key_returns_v(o):
    rng = np.random.default_rng(11)
    q, k, v = _rand64(rng, 1, 4, 8), _rand64(rng, 1, 2, 8), _rand64(rng, 1, 2, 8)
    out = o.ref_contiguous_attention(q, k, v, 0.3, np.array([0]))
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], v[0, h // 2])


def pin_uniform_scores_give_mean(o):
    rng = np.random.default_rng(12)
    lk = 7
    q = np.zeros((3, 2, 8))
    k, v = _rand64(rng, lk, 1, 8), _rand64(rng, lk, 1, 8)
    pos = np.array([0, 3, 6])
    out = o.ref_contiguous_attention(q, k, v, 1.0, pos)
    for i, p in enumerate(pos):
        for h in range(2):
            np.testing.assert_allclose(out[i, h], v[:p + 1, 0].mean(axis=0), rtol=0, atol=1e-14)


def pin_needle(o):
    rng = np.random.default_rng(13)
    lk, d = 40, 16
    qv = rng.standard_normal(d)
    qv /= np.linalg.norm(qv)
    k = np.zeros((lk, 1, d))
    needle = 23
    k[needle, 0] = 2000.0 * qv
    v = rng.integers(-8, 8, (lk, 1, d)).astype(np.float64)
    out = o.ref_contiguous_attention(qv[None, None, :], k, v, 1.0, np.array([lk - 1]))
    np.testing.assert_array_equal(out[0, 0], v[needle, 0])


def pin_gqa_head_mapping(o):
    rng = np.random.default_rng(14)
    hkv, g, d, lk = 3, 4, 8, 9
    q = _rand64(rng, 2, hkv * g, d)
    k = _rand64(rng, lk, hkv, d)
    v = np.empty((lk, hkv, d))
    for j in range(hkv):
        v[:, j, :] = j + 1.0
    out = o.ref_contiguous_attention(q, k, v, 0.5, np.array([4, 8]))
    for h in range(hkv * g):
        np.testing.assert_allclose(out[:, h, :], h // g + 1.0, rtol=1e-14)


def pin_scale_power_of_two(o):
    rng = np.random.default_rng(15)
    q, k, v = _rand64(rng, 5, 2, 8), _rand64(rng, 6, 2, 8), _rand64(rng, 6, 2, 8)
    pos = np.array([1, 2, 3, 4, 5])
    a = o.ref_contiguous_attention(q, k, v, 0.25, pos)
    b = o.ref_contiguous_attention(2.0 * q, k, v, 0.125, pos)
    np.testing.assert_array_equal(a, b)
    c = o.ref_contiguous_attention(q, k, v, 0.5, pos)
    assert np.abs(a - c).max() > 1e-3     # the scale matters


# ------------------------------------------------- library routine (torch SDPA)

def pin_contiguous_vs_torch_sdpa(o):
    rng = np.random.default_rng(16)
    for hq, hkv, d, lq, lk in [(4, 4, 16, 5, 9), (8, 2, 32, 7, 20), (6, 1, 8, 1, 33)]:
        q, k, v = _rand64(rng, lq, hq, d), _rand64(rng, lk, hkv, d), _rand64(rng, lk, hkv, d)
        pos = np.sort(rng.choice(lk, lq, replace=False))
        got = o.ref_contiguous_attention(q, k, v, 1 / math.sqrt(d), pos)
        want = _sdpa64(q, k, v, 1 / math.sqrt(d), pos)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def pin_causality(o):
    rng = np.random.default_rng(17)
    q, k, v = _rand64(rng, 6, 2, 8), _rand64(rng, 6, 1, 8), _rand64(rng, 6, 1, 8)
    pos = np.arange(6)
    base = o.ref_contiguous_attention(q, k, v, 0.4, pos)
    k2, v2 = k.copy(), v.copy()
    k2[4] += 3.0
    v2[4] -= 5.0
    pert = o.ref_contiguous_attention(q, k2, v2, 0.4, pos)
    np.testing.assert_array_equal(base[:4], pert[:4])     # rows before 4 cannot see it
    assert np.abs(base[4] - pert[4]).min() > 0            # row 4 sees its own key


# ---------------------------------------------------- paging and brute force

def _concat_blocks(pool, table_row, n):
    """Brute force: concatenate the sequence's whole blocks in table order,
    then cut to ``n`` tokens."""
    parts = [pool[int(b)] for b in table_row if b >= 0]
    return np.concatenate(parts, axis=0)[:n]


def _small_decode(seed=21, dtype="f16", hq=4, hkv=2, d=32, lens=(1, 15, 16, 17, 40, 0, 33),
                  write_last=True, block_size=16):
    return make_decode_case(name="pin", seed=seed, dtype=dtype, num_q_heads=hq,
                            num_kv_heads=hkv, head_dim=d, seq_lens=list(lens),
                            num_blocks=384 // block_size, max_blocks_per_seq=64 // block_size,
                            scale=1 / math.sqrt(d), write_last=write_last, block_size=block_size)


def pin_paged_decode_equals_contiguous(o):
    for dtype in ("f16", "bf16"):
        c = _small_decode(dtype=dtype)
        kc, vc = o.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
        got = o.ref_decode(c.q, kc, vc, c.block_tables, c.seq_lens, c.scale, dtype)
        for b in range(c.num_seqs):
            n = int(c.seq_lens[b])
            if n == 0:
                np.testing.assert_array_equal(got[b], 0.0)
                continue
            k = o.bits_to_float64(_concat_blocks(kc, c.block_tables[b], n), dtype)
            v = o.bits_to_float64(_concat_blocks(vc, c.block_tables[b], n), dtype)
            assert np.isfinite(k).all() and np.isfinite(v).all()
            q = o.bits_to_float64(c.q[b], dtype)[None]
            want = _sdpa64(q, k, v, c.scale, np.array([n - 1]))[0]
            np.testing.assert_allclose(got[b], want, rtol=0, atol=1e-12)


def pin_block_size_32(o):
    """With 32-token blocks (the other usual size) paged decode is still plain
    attention over the sequence's tokens, and decode and prefill give exactly
    the results of the 16-token layout of the same tokens."""
    for dtype in ("f16", "bf16"):
        c16, c32 = (_small_decode(dtype=dtype, block_size=bs) for bs in (16, 32))
        assert c32.k_cache.shape[1] == 32
        outs = []
        for c in (c16, c32):
            kc, vc = o.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
            outs.append(o.ref_decode(c.q, kc, vc, c.block_tables, c.seq_lens, c.scale, dtype))
        np.testing.assert_array_equal(outs[0], outs[1])
        for b in range(c32.num_seqs):
            n = int(c32.seq_lens[b])
            if n == 0:
                continue
            k = o.bits_to_float64(_concat_blocks(kc, c32.block_tables[b], n), dtype)
            v = o.bits_to_float64(_concat_blocks(vc, c32.block_tables[b], n), dtype)
            q = o.bits_to_float64(c32.q[b], dtype)[None]
            want = _sdpa64(q, k, v, c32.scale, np.array([n - 1]))[0]
            np.testing.assert_allclose(outs[1][b], want, rtol=0, atol=1e-12)
    pre = []
    for bs in (16, 32):
        c = make_prefill_case(name="pin", seed=32, dtype="bf16", num_q_heads=4, num_kv_heads=2,
                              head_dim=16, q_lens=[5, 0, 40, 1], ctx_lens=[31, 3, 16, 33],
                              scale=0.25, extra_blocks=1, block_size=bs)
        kc, vc = o.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
        pre.append(o.ref_prefill_paged(c.q, kc, vc, c.block_tables, c.ctx_lens,
                                       c.query_start_loc, c.scale, "bf16"))
    np.testing.assert_array_equal(pre[0], pre[1])


def pin_block_permutation_invariance(o):
    c = _small_decode(write_last=False, seed=22)
    base = o.ref_decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, c.scale, c.dtype)
    rng = np.random.default_rng(5)
    perm = rng.permutation(c.num_blocks)       # old block i -> new block perm[i]
    kc = np.empty_like(c.k_cache)
    vc = np.empty_like(c.v_cache)
    kc[perm] = c.k_cache
    vc[perm] = c.v_cache
    tables = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    moved = o.ref_decode(c.q, kc, vc, tables, c.seq_lens, c.scale, c.dtype)
    np.testing.assert_array_equal(base, moved)


def pin_shared_prefix_equals_private(o):
    c = make_decode_case(name="pin", seed=23, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                         head_dim=16, seq_lens=[20, 64, 70, 33, 100, 31], num_blocks=40,
                         max_blocks_per_seq=7, scale=0.25, write_last=False, share_group=3,
                         share_tokens=32)
    assert (c.block_tables[0, :2] == c.block_tables[1, :2]).all()
    shared = o.ref_decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, c.scale, "bf16")
    # give every sequence private copies of its blocks in a bigger pool
    nb = int((c.block_tables >= 0).sum())
    kc = np.empty((nb,) + c.k_cache.shape[1:], np.uint16)
    vc = np.empty_like(kc)
    tables = np.full_like(c.block_tables, -1)
    cur = 0
    for b in range(c.num_seqs):
        for j, blk in enumerate(c.block_tables[b]):
            if blk < 0:
                break
            kc[cur], vc[cur] = c.k_cache[blk], c.v_cache[blk]
            tables[b, j] = cur
            cur += 1
    private = o.ref_decode(c.q, kc, vc, tables, c.seq_lens, c.scale, "bf16")
    np.testing.assert_array_equal(shared, private)


def pin_reshape_semantics(o):
    rng = np.random.default_rng(24)
    kc = normal_bits(rng, (4, 16, 2, 8), "f16")
    vc = normal_bits(rng, (4, 16, 2, 8), "f16")
    key = normal_bits(rng, (3, 2, 8), "f16")
    val = normal_bits(rng, (3, 2, 8), "f16")
    slots = np.array([37, -1, 5], np.int64)
    nk, nv = o.ref_reshape_and_cache(key, val, kc, vc, slots)
    np.testing.assert_array_equal(nk[2, 5], key[0])
    np.testing.assert_array_equal(nv[0, 5], val[2])
    changed = np.argwhere((nk != kc).any(axis=(2, 3)))
    assert {tuple(x) for x in changed} <= {(2, 5), (0, 5)}
    np.testing.assert_array_equal(kc, o.ref_reshape_and_cache(key[:0], val[:0], kc, vc, slots[:0])[0])
    for bad in ([64, 0, 1], [5, 5, -1]):
        try:
            o.ref_reshape_and_cache(key, val, kc, vc, np.array(bad, np.int64))
        except (IndexError, ValueError):
            pass
        else:
            raise AssertionError(f"slots {bad} accepted")


def pin_copy_on_write_fork_golden(o):
    """Fork by copy-on-write, worked by hand: after the block copy and the write,
    sequence a still reads the old tokens and sequence b reads its new one."""
    g = _golden("copy_on_write_fork.json")
    nb, bs = g["num_blocks"], g["block_size"]
    rng = np.random.default_rng(51)
    kc = normal_bits(rng, (nb, bs, 1, 8), "f16")
    vc = normal_bits(rng, (nb, bs, 1, 8), "f16")
    kc2, vc2 = o.ref_copy_blocks(kc, vc, np.array(g["copy_pairs"], np.int64))
    src, dst = g["copy_pairs"][0]
    np.testing.assert_array_equal(kc2[dst], kc[src])
    np.testing.assert_array_equal(vc2[dst], vc[src])
    untouched = [b for b in range(nb) if b != dst]
    np.testing.assert_array_equal(kc2[untouched], kc[untouched])
    new_k = normal_bits(rng, (1, 1, 8), "f16")
    kc3, vc3 = o.ref_reshape_and_cache(new_k, new_k, kc2, vc2, np.array([g["fork_slot_b"]], np.int64))
    ta, tb = np.array(g["table_a"]), np.array(g["table_b_after"])
    n = g["tokens"]
    a_k = o.gather_tokens(kc3, ta, n)
    b_k = o.gather_tokens(kc3, tb, n)
    np.testing.assert_array_equal(a_k, o.gather_tokens(kc, ta, n))       # a unchanged
    np.testing.assert_array_equal(b_k[:g["write_token_b"]], a_k[:g["write_token_b"]])
    np.testing.assert_array_equal(b_k[g["write_token_b"]], new_k[0])
    assert g["shared_slot_b"] == ta[g["write_token_b"] // bs] * bs + g["write_token_b"] % bs
    for bad in ([[1, 6], [2, 6]], [[1, 6], [6, 3]], [[1, 9]]):
        try:
            o.ref_copy_blocks(kc, vc, np.array(bad, np.int64))
        except (ValueError, IndexError):
            pass
        else:
            raise AssertionError(f"pairs {bad} accepted")
    same, _ = o.ref_copy_blocks(kc, vc, np.array([[-1, 3], [2, -1]], np.int64))
    np.testing.assert_array_equal(same, kc)                                # negative entries skip


# ------------------------------------------- multi-query (verification) decode

def _multi_case(seed=25, dtype="bf16", nq=4, lens=(1, 3, 4, 5, 16, 17, 40, 33, 0), hq=8, hkv=2, d=16):
    """A decode case whose sequences carry ``nq`` new queries each."""
    c = make_decode_case(name="pin-multi", seed=seed, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                         head_dim=d, seq_lens=list(lens), num_blocks=30, max_blocks_per_seq=4,
                         scale=0.3, write_last=False)
    q = normal_bits(np.random.default_rng(seed + 1), (len(lens), nq, hq, d), dtype)
    return c, q


def pin_multi_query_equals_chunked_prefill(o):
    """Q queries at positions n-Q .. n-1 are a prefill chunk of Q rows over a
    context of n-Q cached tokens (sequences with n >= Q)."""
    c, q = _multi_case()
    nq = q.shape[1]
    got = o.ref_decode_multi(q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, c.scale, "bf16")
    keep = [b for b in range(c.num_seqs) if int(c.seq_lens[b]) >= nq]
    ctx = np.array([int(c.seq_lens[b]) - nq for b in keep], np.int32)
    qsl = np.arange(len(keep) + 1, dtype=np.int32) * nq
    pre = o.ref_prefill_paged(q[keep].reshape(-1, *q.shape[2:]), c.k_cache, c.v_cache,
                              c.block_tables[keep], ctx, qsl, c.scale, "bf16")
    np.testing.assert_allclose(got[keep].reshape(pre.shape), pre, rtol=0, atol=1e-13)


def pin_multi_query_rows_are_rolled_back_decodes(o):
    """Row j equals a plain decode of the same query with seq_len n - Q + j + 1:
    rejecting drafts is just a shorter sequence; rows before the first token
    are zero; one query per sequence is plain decode."""
    c, q = _multi_case(seed=26, dtype="f16")
    nq = q.shape[1]
    got = o.ref_decode_multi(q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, c.scale, "f16")
    for b in range(c.num_seqs):
        n = int(c.seq_lens[b])
        for j in range(nq):
            lim = n - nq + j + 1
            if lim <= 0:
                np.testing.assert_array_equal(got[b, j], 0.0)
                continue
            dec = o.ref_decode(q[b:b + 1, j], c.k_cache, c.v_cache, c.block_tables[b:b + 1],
                               np.array([lim]), c.scale, "f16")
            np.testing.assert_allclose(got[b, j], dec[0], rtol=0, atol=1e-13)
    one = o.ref_decode_multi(q[:, :1], c.k_cache, c.v_cache, c.block_tables, c.seq_lens, c.scale, "f16")
    np.testing.assert_array_equal(one[:, 0], o.ref_decode(q[:, 0], c.k_cache, c.v_cache, c.block_tables,
                                                          c.seq_lens, c.scale, "f16"))


# ------------------------------------------------------------ chunked prefill

def _small_prefill(seed=31, q_lens=(5, 0, 17, 1, 33), ctx=(0, 9, 20, 15, 40)):
    return make_prefill_case(name="pin", seed=seed, dtype="bf16", num_q_heads=6, num_kv_heads=2,
                             head_dim=16, q_lens=list(q_lens), ctx_lens=list(ctx), scale=0.25,
                             extra_blocks=3)


def pin_prefill_equals_sdpa(o):
    c = _small_prefill()
    kc, vc = o.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    got = o.ref_prefill_paged(c.q, kc, vc, c.block_tables, c.ctx_lens, c.query_start_loc,
                              c.scale, "bf16")
    for b in range(c.num_seqs):
        lo, hi = int(c.query_start_loc[b]), int(c.query_start_loc[b + 1])
        if hi == lo:
            continue
        ctx = int(c.ctx_lens[b])
        n = ctx + hi - lo
        k = o.bits_to_float64(_concat_blocks(kc, c.block_tables[b], n), "bf16")
        v = o.bits_to_float64(_concat_blocks(vc, c.block_tables[b], n), "bf16")
        assert np.isfinite(k).all()
        q = o.bits_to_float64(c.q[lo:hi], "bf16")
        want = _sdpa64(q, k, v, c.scale, ctx + np.arange(hi - lo))
        np.testing.assert_allclose(got[lo:hi], want, rtol=0, atol=1e-12)


def pin_prefill_no_context_is_plain_causal(o):
    c = _small_prefill(seed=32, q_lens=(12, 30), ctx=(0, 0))
    kc, vc = o.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    got = o.ref_prefill_paged(c.q, kc, vc, c.block_tables, c.ctx_lens, c.query_start_loc,
                              c.scale, "bf16")
    for b in range(2):
        lo, hi = int(c.query_start_loc[b]), int(c.query_start_loc[b + 1])
        q = torch.from_numpy(o.bits_to_float64(c.q[lo:hi], "bf16").transpose(1, 0, 2).copy())[None]
        k = torch.from_numpy(o.bits_to_float64(c.key[lo:hi], "bf16").transpose(1, 0, 2).copy())[None]
        v = torch.from_numpy(o.bits_to_float64(c.value[lo:hi], "bf16").transpose(1, 0, 2).copy())[None]
        want = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, is_causal=True, scale=c.scale, enable_gqa=True)[0].numpy().transpose(1, 0, 2)
        np.testing.assert_allclose(got[lo:hi], want, rtol=0, atol=1e-12)


def pin_prefill_chunks_equal_whole(o):
    """Two chunks (the second with the first as cached context) equal one."""
    c = _small_prefill(seed=33, q_lens=(29,), ctx=(7,))
    kc, vc = o.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    whole = o.ref_prefill_paged(c.q, kc, vc, c.block_tables, c.ctx_lens, c.query_start_loc,
                                c.scale, "bf16")
    split = 11
    first = o.ref_prefill_paged(c.q[:split], kc, vc, c.block_tables, c.ctx_lens,
                                np.array([0, split], np.int32), c.scale, "bf16")
    second = o.ref_prefill_paged(c.q[split:], kc, vc, c.block_tables, c.ctx_lens + split,
                                 np.array([0, 29 - split], np.int32), c.scale, "bf16")
    # different row counts may take different BLAS summation orders
    np.testing.assert_allclose(np.concatenate([first, second]), whole, rtol=0, atol=1e-13)


def pin_prefill_row_equals_decode(o):
    c = _small_prefill(seed=34, q_lens=(9, 4), ctx=(21, 0))
    kc, vc = o.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    got = o.ref_prefill_paged(c.q, kc, vc, c.block_tables, c.ctx_lens, c.query_start_loc,
                              c.scale, "bf16")
    for b, row in [(0, 8), (0, 0), (1, 3)]:
        r = int(c.query_start_loc[b]) + row
        dec = o.ref_decode(c.q[r:r + 1], kc, vc, c.block_tables[b:b + 1],
                           np.array([int(c.ctx_lens[b]) + row + 1]), c.scale, "bf16")
        np.testing.assert_allclose(dec[0], got[r], rtol=0, atol=1e-13)


# ------------------------------------------------------ split-KV merge algebra

def pin_split_merge(o):
    rng = np.random.default_rng(41)
    hq, hkv, d, n = 8, 2, 16, 97
    q = _rand64(rng, hq, d)
    k, v = _rand64(rng, n, hkv, d) * 2.0, _rand64(rng, n, hkv, d)
    whole = o.ref_contiguous_attention(q[None], k, v, 0.3, np.array([n - 1]))[0]
    for part in (1, 16, 30, 64, 97):
        bounds = list(range(0, n, part)) + [n]
        states = [o.ref_partition_state(q, k, v, 0.3, a, b) for a, b in zip(bounds[:-1], bounds[1:])]
        ms, ls, accs = (np.stack(x) for x in zip(*states))
        merged = o.ref_merge_partitions(ms, ls, accs)
        np.testing.assert_allclose(merged, whole, rtol=0, atol=1e-12)
    # a single partition's state normalises to the answer directly
    m, l, acc = o.ref_partition_state(q, k, v, 0.3, 0, n)
    np.testing.assert_allclose(acc / l[:, None], whole, rtol=0, atol=1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
