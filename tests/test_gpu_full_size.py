"""Parity at the workloads' full sizes, in the launch configuration the bench
times (default partition length).  The 16-bit decode and prefill workloads
are checked on EVERY output against the float64 oracle (one pass per
sequence), so a work item skipped or computed twice anywhere in the grid --
including the prefill work-order search -- cannot hide behind a sample.  The
FP8 workloads, whose oracle quantises every checked token on the host, and
draft verification are checked on at least 16 sequences each (4 of the 8
64K-token sequences of the long-context workload), spanning the shortest,
the longest and the first and last of each batch."""

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


def _every_sequence_decode(c, flags=0):
    g = DecodeOnGPU(c)
    if len(c.slot_mapping):
        _written_rows_exact(g, c)
        kc, vc = oracle.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    else:
        kc, vc = c.k_cache, c.v_cache
    out = host_f64(g.decode(flags=flags))
    worst = 0.0
    for b in range(c.num_seqs):
        ref = oracle.ref_decode_one(c.q[b], kc, vc, c.block_tables[b], int(c.seq_lens[b]),
                                    c.scale, c.dtype)
        worst = max(worst, assert_close(out[b], ref, c.dtype,
                                        f"{c.name} seq {b} (len {int(c.seq_lens[b])})"))
    print(f"{c.name}: {c.num_seqs} sequences, max-abs error {worst:.3e}")


def _pick(lens, count):
    """`count` sequences: first, last, longest, shortest, the rest evenly spread."""
    lens = np.asarray(lens)
    keep = {0, len(lens) - 1, int(lens.argmax()), int(lens.argmin())}
    for i in np.linspace(0, len(lens) - 1, count).astype(int):
        if len(keep) >= count:
            break
        keep.add(int(i))
    return sorted(keep)


def test_full_llama2_7b_layer_decode():
    _every_sequence_decode(decode_llama2_7b_layer())


def test_full_gqa_shared_prefix_decode():
    _every_sequence_decode(decode_gqa_shared_prefix())


def test_full_gqa_shared_prefix_decode_sequence_groups():
    """With PA_DECODE_SHARED_PREFIX: waves of 4 sequences read each shared prefix block once."""
    import paged_kv_cache_24_amd as pa
    _every_sequence_decode(decode_gqa_shared_prefix(), flags=pa.PA_DECODE_SHARED_PREFIX)


def test_full_long_context_decode():
    _every_sequence_decode(decode_long_context())


def test_full_chunked_prefill():
    """Every row of all 16 sequences (8192 rows x 32 heads)."""
    c = prefill_chunked()
    g = PrefillOnGPU(c)
    _written_rows_exact(g, c)
    kc, vc = oracle.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    out = host_f64(g.prefill())
    worst = 0.0
    for b in range(c.num_seqs):
        L = int(c.q_lens[b])
        if L == 0:
            continue
        lo = int(c.query_start_loc[b])
        ref = oracle.ref_prefill_rows(c.q, kc, vc, c.block_tables[b], int(c.ctx_lens[b]), lo,
                                      np.arange(L), c.scale, c.dtype)
        worst = max(worst, assert_close(out[lo:lo + L], ref, c.dtype,
                                        f"prefill seq {b} (ctx {int(c.ctx_lens[b])}, {L} rows)"))
    print(f"prefill_chunked: {c.num_tokens} rows, max-abs error {worst:.3e}")


# ---- FP8 cache (E4M3 codes, one scale per token and kv head) and draft
# verification, at the same full sizes.  The oracle quantises only the checked
# sequences' tokens from the 16-bit k/v (never from the GPU pools), checks the
# GPU pools bit-exactly at those slots, and attends over its own pools.

def _fp8_pools(g, slots_wanted):
    """Oracle FP8 pools holding exactly the given slots, plus the GPU pool rows there."""
    sel = np.flatnonzero(np.isin(g.slots_np, slots_wanted))
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
    wanted = np.unique(np.concatenate([_seq_slots(c.block_tables[b], int(c.seq_lens[b]))
                                       for b in samples]))
    kc, vc, ks, vs = _fp8_pools(g, wanted)
    sel = np.asarray(samples)
    ref = oracle.ref_decode_fp8(c.q[sel], kc, vc, ks, vs, c.block_tables[sel], c.seq_lens[sel],
                                c.scale, c.dtype)
    worst = 0.0
    for i, b in enumerate(samples):
        worst = max(worst, assert_close(out[b], ref[i], c.dtype,
                                        f"{c.name} fp8 seq {b} (len {int(c.seq_lens[b])})"))
    print(f"{c.name} fp8: {len(samples)} sequences, max-abs error {worst:.3e}")


def test_full_llama2_7b_layer_decode_fp8():
    import paged_kv_cache_24_amd as pa
    c = decode_llama2_7b_layer()
    _sampled_decode_fp8(c, _pick(c.seq_lens, 16), flags=pa.PA_DECODE_STREAM_KV)


def test_full_gqa_shared_prefix_decode_fp8():
    c = decode_gqa_shared_prefix()
    _sampled_decode_fp8(c, _pick(c.seq_lens, 16))


def test_full_gqa_shared_prefix_decode_fp8_sequence_groups():
    import paged_kv_cache_24_amd as pa
    c = decode_gqa_shared_prefix()
    _sampled_decode_fp8(c, _pick(c.seq_lens, 16), flags=pa.PA_DECODE_SHARED_PREFIX)


def test_full_long_context_decode_fp8():
    import paged_kv_cache_24_amd as pa
    _sampled_decode_fp8(decode_long_context(), [0, 2, 5, 7], flags=pa.PA_DECODE_STREAM_KV)


def test_full_chunked_prefill_fp8():
    """Every row of all 16 sequences over the FP8 cache."""
    from gpu_helpers import Fp8PrefillOnGPU
    c = prefill_chunked()
    g = Fp8PrefillOnGPU(c)
    g.write()
    out = host_f64(g.prefill())
    assert np.isfinite(out).all()
    kc, vc, ks, vs = _fp8_pools(g, g.slots_np)
    worst = 0.0
    for b in range(c.num_seqs):
        L, ctx = int(c.q_lens[b]), int(c.ctx_lens[b])
        if L == 0:
            continue
        lo = int(c.query_start_loc[b])
        ref = oracle.ref_prefill_rows_fp8(c.q, kc, vc, ks, vs, c.block_tables[b], ctx, lo,
                                          np.arange(L), c.scale, c.dtype)
        worst = max(worst, assert_close(out[lo:lo + L], ref, c.dtype,
                                        f"fp8 prefill seq {b} (ctx {ctx}, {L} rows)"))
    print(f"prefill_chunked fp8: {c.num_tokens} rows, max-abs error {worst:.3e}")


def test_full_llama2_7b_layer_verify():
    """Four queries per sequence (three drafts and the last accepted token) over
    the LLaMA-shaped layer, with the library's default partition: every
    sequence."""
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
    worst = 0.0
    for b in range(c.num_seqs):
        ref = oracle.ref_decode_multi(qbits[b:b + 1], kc, vc, c.block_tables[b:b + 1],
                                      c.seq_lens[b:b + 1], c.scale, c.dtype)[0]
        worst = max(worst, assert_close(got[b], ref, c.dtype,
                                        f"verify seq {b} (len {int(c.seq_lens[b])})"))
    print(f"verification: {c.num_seqs} sequences x {nq} queries, max-abs error {worst:.3e}")
