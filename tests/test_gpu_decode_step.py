"""pa_decode_step: the decode step's cache write done inside the decode
kernels.  Against the oracle (its cache write with the table-derived slots,
then its decode) and against the separate calls (pa_reshape_and_cache +
pa_decode): the pools bit for bit, the outputs to the decode tolerance (the
newest key joins the softmax in its own step).  Covers the vector path (1 and
2 q heads per kv head, head_dim 64 and 128), the matrix-core path (3..24 q
heads per kv head, head chunks), 16- and 32-token blocks, fixed partitions and
the balanced split, sequences of 0 and 1 tokens, a newest token that opens a
block, and a newest token whose block lies outside the pool (not written)."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DecodeOnGPU, TOL, assert_close, dev_bits, dev_int, host_bits, host_f64, require_gpu
from workloads import decode_gqa_shared_prefix, make_decode_case, normal_bits

pytestmark = pytest.mark.gpu

LENS = [0, 1, 2, 15, 16, 17, 32, 33, 64, 100, 257, 300]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import paged_kv_cache_24_amd  # noqa: F401


def _table_slots(c):
    n = c.seq_lens.astype(np.int64)
    bs = c.block_size
    slots = np.full(c.num_seqs, -1, np.int64)
    for b in range(c.num_seqs):
        if n[b] > 0:
            e = int(c.block_tables[b, (n[b] - 1) // bs])
            if 0 <= e < c.num_blocks:
                slots[b] = e * bs + (n[b] - 1) % bs
    return slots


def _step_rows(c):
    """key / value rows for every sequence: the workload's newest-token rows (one
    per non-empty sequence, in order), zeros for the empty ones (never read)."""
    shape = (c.num_seqs, c.num_kv_heads, c.head_dim)
    k, v = np.zeros(shape, np.uint16), np.zeros(shape, np.uint16)
    live = np.flatnonzero(c.seq_lens > 0)
    k[live], v[live] = c.key, c.value
    return dev_bits(k, c.dtype), dev_bits(v, c.dtype)


def _run(c, part, flags=0, tables=None):
    """(out of the step, its K and V pools, out of the separate calls)"""
    import paged_kv_cache_24_amd as pa
    g1, g2 = DecodeOnGPU(c), DecodeOnGPU(c)
    if tables is not None:
        g1.tables = dev_int(tables)
        g2.tables = dev_int(tables)
    key, value = _step_rows(c)
    out1 = torch.empty_like(g1.q)
    pa.pa_decode_step(out1, g1.q, key, value, g1.k_cache, g1.v_cache, g1.tables, g1.lens, c.scale, part,
                      flags=flags)
    g2.write()
    out2 = g2.decode(partition_tokens=part, flags=flags)
    torch.cuda.synchronize()
    return host_f64(out1), host_bits(g1.k_cache), host_bits(g1.v_cache), host_f64(out2)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 128), (8, 4, 64), (8, 2, 128), (16, 2, 128), (48, 2, 128),
                                      (4, 1, 64)])
@pytest.mark.parametrize("bs", [16, 32])
def test_step_matches_oracle_and_separate_calls(dtype, hq, hkv, d, bs):
    c = make_decode_case(name=f"step-{dtype}-{hq}-{hkv}-{d}-{bs}", seed=1000 + hq + d + bs, dtype=dtype,
                         num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seq_lens=LENS, num_blocks=80,
                         max_blocks_per_seq=320 // bs, scale=1 / math.sqrt(d), write_last=True, block_size=bs)
    slots = _table_slots(c)
    assert (slots[c.seq_lens > 0] == c.slot_mapping).all()   # the workload's writes: the newest tokens
    kc, vc = oracle.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    ref = oracle.ref_decode(c.q, kc, vc, c.block_tables, c.seq_lens, c.scale, dtype)
    for part in (0, 16, 64, -1):
        out, k1, v1, out2 = _run(c, part)
        np.testing.assert_array_equal(k1, kc, err_msg=f"K pool, partition {part}")
        np.testing.assert_array_equal(v1, vc, err_msg=f"V pool, partition {part}")
        assert_close(out, ref, dtype, f"{c.name} partition={part}")
        # both within TOL of the oracle; between them the rounding of one 16-bit output may differ
        assert np.abs(out - out2).max() <= 2 * TOL[dtype]
        assert (out[c.seq_lens == 0] == 0).all()


def test_newest_block_outside_the_pool_is_not_written():
    c = make_decode_case(name="step-bad", seed=1077, dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128,
                         seq_lens=[40, 17, 33], num_blocks=12, max_blocks_per_seq=4, scale=0.1, write_last=True)
    tables = c.block_tables.copy()
    tables[1, 1] = c.num_blocks + 5           # the block of sequence 1's newest token (position 16)
    tables[2, 2] = -1                         # and of sequence 2's (position 32)
    out, k1, v1, _ = _run(c, 0, tables=tables)
    kc, vc = oracle.ref_reshape_and_cache(c.key[:1], c.value[:1], c.k_cache, c.v_cache, c.slot_mapping[:1])
    np.testing.assert_array_equal(k1, kc)     # only sequence 0's row was written
    np.testing.assert_array_equal(v1, vc)
    ref = oracle.ref_decode(c.q[:1], kc, vc, tables[:1], c.seq_lens[:1], c.scale, "bf16")
    assert_close(out[:1], ref, "bf16", "sequence 0")
    assert np.isfinite(out).all()


def test_step_with_sequence_groups_equals_separate_calls_bit_exact():
    """PA_DECODE_SHARED_PREFIX: the write runs first as its own kernel, then the groups."""
    import paged_kv_cache_24_amd as pa
    # a newest token for every sequence, in a block of its own past the 256-token prefix
    base = decode_gqa_shared_prefix(batch=24, max_len=1024, min_len=16, group=4, prefix=256)
    lens = np.maximum(base.seq_lens, 257).astype(np.int32)
    c = make_decode_case(name="step-groups", seed=1078, dtype="bf16", num_q_heads=32, num_kv_heads=8,
                         head_dim=128, seq_lens=lens, num_blocks=int(sum((x + 15) // 16 for x in lens)) + 8,
                         max_blocks_per_seq=64, scale=1 / math.sqrt(128), write_last=False, share_group=4,
                         share_tokens=256)
    g1, g2 = DecodeOnGPU(c), DecodeOnGPU(c)
    rng = np.random.default_rng(1079)
    key = dev_bits(normal_bits(rng, (c.num_seqs, 8, 128), "bf16"), "bf16")
    value = dev_bits(normal_bits(rng, (c.num_seqs, 8, 128), "bf16"), "bf16")
    flags = pa.PA_DECODE_SHARED_PREFIX
    out1 = torch.empty_like(g1.q)
    pa.pa_decode_step(out1, g1.q, key, value, g1.k_cache, g1.v_cache, g1.tables, g1.lens, c.scale, flags=flags)
    pa.pa_reshape_and_cache(key, value, g2.k_cache, g2.v_cache, dev_int(_table_slots(c), torch.int64))
    out2 = g2.decode(flags=flags)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(g1.k_cache), host_bits(g2.k_cache))
    np.testing.assert_array_equal(host_bits(out1), host_bits(out2))


def test_partitions_step_then_merge_equals_step():
    import paged_kv_cache_24_amd as pa
    c = make_decode_case(name="step-phases", seed=1080, dtype="f16", num_q_heads=32, num_kv_heads=32,
                         head_dim=128, seq_lens=[700, 1, 0, 129, 2048, 64], num_blocks=200,
                         max_blocks_per_seq=128, scale=1 / math.sqrt(128), write_last=True)
    g1, g2 = DecodeOnGPU(c), DecodeOnGPU(c)
    key, value = _step_rows(c)
    need = pa.pa_decode_workspace_size(c.num_seqs, 32, 32, 128, 16, 128, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out1 = torch.empty_like(g1.q)
    pa.pa_decode_step(out1, g1.q, key, value, g1.k_cache, g1.v_cache, g1.tables, g1.lens, c.scale,
                      workspace=ws)
    out2 = torch.empty_like(g2.q)
    pa.pa_decode_partitions_step(out2, g2.q, key, value, g2.k_cache, g2.v_cache, g2.tables, g2.lens,
                                 c.scale, ws)
    pa.pa_decode_merge(out2, g2.lens, 32, 128, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(out1), host_bits(out2))
    np.testing.assert_array_equal(host_bits(g1.k_cache), host_bits(g2.k_cache))
