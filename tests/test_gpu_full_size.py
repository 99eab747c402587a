"""Parity at the workloads' full sizes, in the launch configuration the bench
times (default partition length), checked on sampled outputs the oracle
computes one sequence at a time: the 16-bit decode and prefill workloads, the
same over the FP8 cache, and draft verification on the LLaMA-shaped layer."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DecodeOnGPU, PrefillOnGPU, assert_close, host_bits, host_f64, require_gpu
from workloads import (decode_gqa_shared_prefix, decode_llama2_7b_layer, decode_long_context,
                       prefill_chunked)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import paged_kv_cache_24_amd  # noqa: F401


def _written_rows_exact(g, c):
    """After the cache write: exactly the slot rows changed, and they hold the new k/v."""
    before_k = g.k_cache.clone()
    before_v = g.v_cache.clone()
    g.write()
    torch.cuda.synchronize()
    nb = c.k_cache.shape[0]
    for before, after, new in ((before_k, g.k_cache, c.key), (before_v, g.v_cache, c.value)):
        changed = (before.view(torch.int16) != after.view(torch.int16)).flatten(2).any(dim=2)
        got = set(torch.nonzero(changed.flatten()).flatten().cpu().tolist())
        assert got == set(int(s) for s in c.slot_mapping)
        slots = torch.from_numpy(c.slot_mapping).cuda()
        rows = host_bits(after.view(nb * 16, *after.shape[2:])[slots])
        np.testing.assert_array_equal(rows, new)
    del before_k, before_v


def _sampled_decode(c, samples):
    g = DecodeOnGPU(c)
    if len(c.slot_mapping):
        _written_rows_exact(g, c)
        kc, vc = oracle.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    else:
        kc, vc = c.k_cache, c.v_cache
    out = host_f64(g.decode())
    assert np.isfinite(out).all()
    for b in samples:
        ref = oracle.ref_decode_one(c.q[b], kc, vc, c.block_tables[b], int(c.seq_lens[b]),
                                    c.scale, c.dtype)
        assert_close(out[b], ref, c.dtype, f"{c.name} seq {b} (len {int(c.seq_lens[b])})")


def _pick(lens, extra):
    lens = np.asarray(lens)
    return sorted({0, len(lens) - 1, int(lens.argmax()), int(lens.argmin()), *extra})


def test_full_llama2_7b_layer_decode():
    c = decode_llama2_7b_layer()
    _sampled_decode(c, _pick(c.seq_lens, [17, 40]))


def test_full_gqa_shared_prefix_decode():
    c = decode_gqa_shared_prefix()
    _sampled_decode(c, _pick(c.seq_lens, [1, 15, 16, 100, 200]))


def test_full_long_context_decode():
    c = decode_long_context()
    _sampled_decode(c, [0, 5])


def test_full_chunked_prefill():
    c = prefill_chunked()
    g = PrefillOnGPU(c)
    _written_rows_exact(g, c)
    kc, vc = oracle.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    out = host_f64(g.prefill())
    assert np.isfinite(out).all()
    for b in (0, 7, 15):
        L = int(c.q_lens[b])
        rows = np.unique(np.array([0, 1, L // 2, L - 2, L - 1]).clip(0, L - 1))
        lo = int(c.query_start_loc[b])
        ref = oracle.ref_prefill_rows(c.q, kc, vc, c.block_tables[b], int(c.ctx_lens[b]), lo, rows,
                                      c.scale, c.dtype)
        assert_close(out[lo + rows], ref, c.dtype, f"prefill seq {b} rows {rows.tolist()}")


# ---- FP8 cache (E4M3 codes, one scale per token and kv head) and draft
# verification, at the same full sizes.  The oracle quantises only the sampled
# sequences' tokens from the 16-bit k/v (never from the GPU pools), checks the
# GPU pools bit-exactly at those slots, and attends over its own pools.

def _fp8_seq_pools(g, b_slots):
    """Oracle FP8 pools holding exactly the given slots, plus the GPU pool rows there."""
    sel = np.flatnonzero(np.isin(g.slots_np, b_slots))
    kc, vc, ks, vs = oracle.ref_reshape_and_cache_fp8(
        g.key_np[sel], g.value_np[sel], g.codes0, g.codes0, g.scales0, g.scales0,
        g.slots_np[sel], g.case.dtype)
    slots = g.slots_np[sel]
    blk, off = slots // 16, slots % 16
    np.testing.assert_array_equal(g.k_cache.cpu().numpy()[blk, off], kc[blk, off])
    np.testing.assert_array_equal(g.v_cache.cpu().numpy()[blk, off], vc[blk, off])
    np.testing.assert_array_equal(g.k_scales.cpu().numpy()[blk, :, off], ks[blk, :, off])
    np.testing.assert_array_equal(g.v_scales.cpu().numpy()[blk, :, off], vs[blk, :, off])
    return kc, vc, ks, vs


def _seq_slots(table_row, n):
    p = np.arange(n, dtype=np.int64)
    return table_row[p // 16].astype(np.int64) * 16 + p % 16


def _sampled_decode_fp8(c, samples, flags=0):
    from gpu_helpers import Fp8DecodeOnGPU
    g = Fp8DecodeOnGPU(c)
    g.write()
    out = host_f64(g.decode(flags=flags))
    assert np.isfinite(out).all()
    for b in samples:
        n = int(c.seq_lens[b])
        kc, vc, ks, vs = _fp8_seq_pools(g, _seq_slots(c.block_tables[b], n))
        ref = oracle.ref_decode_fp8(c.q[b:b + 1], kc, vc, ks, vs, c.block_tables[b:b + 1],
                                    c.seq_lens[b:b + 1], c.scale, c.dtype)[0]
        assert_close(out[b], ref, c.dtype, f"{c.name} fp8 seq {b} (len {n})")


def test_full_llama2_7b_layer_decode_fp8():
    import paged_kv_cache_24_amd as pa
    c = decode_llama2_7b_layer()
    _sampled_decode_fp8(c, _pick(c.seq_lens, [17]), flags=pa.PA_DECODE_STREAM_KV)


def test_full_gqa_shared_prefix_decode_fp8():
    c = decode_gqa_shared_prefix()
    _sampled_decode_fp8(c, _pick(c.seq_lens, [1, 16, 100]))


def test_full_long_context_decode_fp8():
    import paged_kv_cache_24_amd as pa
    _sampled_decode_fp8(decode_long_context(), [0, 5], flags=pa.PA_DECODE_STREAM_KV)


def test_full_chunked_prefill_fp8():
    from gpu_helpers import Fp8PrefillOnGPU
    c = prefill_chunked()
    g = Fp8PrefillOnGPU(c)
    g.write()
    out = host_f64(g.prefill())
    assert np.isfinite(out).all()
    for b in (0, 15):
        L, ctx = int(c.q_lens[b]), int(c.ctx_lens[b])
        rows = np.unique(np.array([0, L // 2, L - 1]).clip(0, L - 1))
        kc, vc, ks, vs = _fp8_seq_pools(g, _seq_slots(c.block_tables[b], ctx + L))
        lo = int(c.query_start_loc[b])
        ref = oracle.ref_prefill_rows_fp8(c.q, kc, vc, ks, vs, c.block_tables[b], ctx, lo, rows,
                                          c.scale, c.dtype)
        assert_close(out[lo + rows], ref, c.dtype, f"fp8 prefill seq {b} rows {rows.tolist()}")


def test_full_llama2_7b_layer_verify():
    """Four queries per sequence (three drafts and the last accepted token) over
    the LLaMA-shaped layer, with the library's default partition."""
    import paged_kv_cache_24_amd as pa
    c = decode_llama2_7b_layer()
    g = DecodeOnGPU(c)
    g.write()
    kc, vc = oracle.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    nq = 4
    rng = np.random.default_rng(11)
    qb = rng.standard_normal((c.num_seqs, nq, c.num_q_heads, c.head_dim), dtype=np.float32)
    qbits = qb.astype(np.float16).view(np.uint16)
    q = torch.from_numpy(qbits.view(np.float16)).cuda()
    out = torch.empty_like(q)
    need = pa.pa_decode_workspace_size(c.num_seqs * nq, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                       16, c.max_blocks_per_seq, 0)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    pa.pa_decode_multi(out, q, g.k_cache, g.v_cache, g.tables, g.lens, c.scale, 0, ws)
    got = host_f64(out)
    assert np.isfinite(got).all()
    for b in _pick(c.seq_lens, [9]):
        ref = oracle.ref_decode_multi(qbits[b:b + 1], kc, vc, c.block_tables[b:b + 1],
                                      c.seq_lens[b:b + 1], c.scale, c.dtype)[0]
        assert_close(got[b], ref, c.dtype, f"verify seq {b} (len {int(c.seq_lens[b])})")
