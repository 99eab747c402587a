"""GPU parity of chunked prefill (MFMA) against the float64 oracle, and
GPU-side consistency with decode and with chunk splitting."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (DecodeOnGPU, PrefillOnGPU, TOL, assert_close, dev_int, host_bits,
                         host_f64, require_gpu)
from workloads import make_decode_case, make_prefill_case, prefill_chunked

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import paged_kv_cache_24_amd  # noqa: F401


def _run(c):
    g = PrefillOnGPU(c)
    g.write()
    kc, vc = oracle.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    np.testing.assert_array_equal(host_bits(g.k_cache), kc)
    np.testing.assert_array_equal(host_bits(g.v_cache), vc)
    out = host_f64(g.prefill())
    ref = oracle.ref_prefill_paged(c.q, kc, vc, c.block_tables, c.ctx_lens, c.query_start_loc,
                                   c.scale, c.dtype)
    return g, out, ref


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (8, 2), (16, 2), (12, 4), (10, 2), (12, 2),
                                    (14, 2), (16, 1)])
def test_prefill_shapes(dtype, hq, hkv, d):
    q_lens = [0, 1, 17, 64, 130, 5, 33]
    ctx = [3, 0, 40, 0, 100, 16, 250]
    c = make_prefill_case(name=f"prefill-{dtype}-{hq}-{hkv}-d{d}", seed=200 + hq + d, dtype=dtype,
                          num_q_heads=hq, num_kv_heads=hkv, head_dim=d, q_lens=q_lens,
                          ctx_lens=ctx, scale=1 / math.sqrt(d), extra_blocks=5)
    _, out, ref = _run(c)
    assert_close(out, ref, dtype, c.name)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_head_dim_64_long(dtype):
    """head_dim 64 over many key tiles and every q tile of a long chunk."""
    c = make_prefill_case(name=f"prefill-d64-long-{dtype}", seed=77, dtype=dtype, num_q_heads=32,
                          num_kv_heads=4, head_dim=64, q_lens=[300, 1, 129], ctx_lens=[700, 1500, 0],
                          scale=1 / 8, extra_blocks=3)
    _, out, ref = _run(c)
    assert_close(out, ref, dtype, c.name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(64, 2), (128, 1)])
def test_prefill_large_groups(hq, hkv, d):
    """32 and 128 q heads per kv head: a workgroup then holds 8 / 4 (or 2 / 1)
    positions, the work order still covers every row."""
    c = make_prefill_case(name=f"prefill-group-{hq // hkv}-d{d}", seed=91 + hq + d, dtype="bf16",
                          num_q_heads=hq, num_kv_heads=hkv, head_dim=d, q_lens=[9, 0, 4, 1],
                          ctx_lens=[30, 5, 0, 70], scale=1 / math.sqrt(d), extra_blocks=2)
    _, out, ref = _run(c)
    assert_close(out, ref, "bf16", c.name)


def test_prefill_chunked_reduced():
    c = prefill_chunked(batch=4, new_tokens=600, max_ctx=700)
    _, out, ref = _run(c)
    assert_close(out, ref, "bf16", c.name)


def test_prefill_rows_outside_sequences_untouched():
    c = make_prefill_case(name="gap", seed=31, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                          head_dim=128, q_lens=[20, 9], ctx_lens=[5, 0], scale=0.1)
    g = PrefillOnGPU(c)
    g.write()
    # the second sequence's rows are dropped from query_start_loc: they must stay untouched
    g.qsl = dev_int(np.array([0, 20, 20], np.int32))
    g.out.fill_(3.0)
    out = host_f64(g.prefill())
    assert (out[20:] == 3.0).all()


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_row_matches_decode(d):
    """A prefill row at position p equals decode with seq_len p + 1."""
    c = make_prefill_case(name=f"rowdec-d{d}", seed=32, dtype="bf16", num_q_heads=16, num_kv_heads=4,
                          head_dim=d, q_lens=[50, 7], ctx_lens=[90, 300], scale=0.08)
    g, out, ref = _run(c)
    assert_close(out, ref, "bf16", c.name)
    for b, row in [(0, 0), (0, 49), (1, 6)]:
        r = int(c.query_start_loc[b]) + row
        q1 = g.q[r:r + 1].contiguous()
        out1 = torch.empty_like(q1)
        import paged_kv_cache_24_amd as pa
        lens = dev_int(np.array([int(c.ctx_lens[b]) + row + 1], np.int32))
        pa.pa_decode(out1, q1, g.k_cache, g.v_cache, g.tables[b:b + 1].contiguous(), lens, c.scale)
        assert np.abs(host_f64(out1)[0] - out[r]).max() <= 2 * TOL["bf16"]


def test_prefill_two_chunks_match_one():
    """Chunk 2 reading chunk 1's KV from the cache gives the one-chunk result."""
    c = make_prefill_case(name="chunks", seed=33, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                          head_dim=128, q_lens=[200], ctx_lens=[37], scale=0.1)
    g, whole, ref = _run(c)
    import paged_kv_cache_24_amd as pa
    split = 77
    out1 = torch.zeros_like(g.q[:split])
    pa.pa_prefill_paged(out1, g.q[:split].contiguous(), g.k_cache, g.v_cache, g.tables, g.ctx,
                        dev_int(np.array([0, split], np.int32)), c.scale, split)
    out2 = torch.zeros_like(g.q[split:])
    pa.pa_prefill_paged(out2, g.q[split:].contiguous(), g.k_cache, g.v_cache, g.tables,
                        g.ctx + split, dev_int(np.array([0, 200 - split], np.int32)), c.scale,
                        200 - split)
    both = np.concatenate([host_f64(out1), host_f64(out2)])
    assert_close(both, ref, "bf16", "two chunks")
    assert np.abs(both - whole).max() <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_long_context(dtype):
    """A context of ~9000 keys: more than two 64-tile chunks of block ids, so
    the kernel refills its cached ids twice while it runs."""
    c = make_prefill_case(name=f"long-{dtype}", seed=34, dtype=dtype, num_q_heads=8,
                          num_kv_heads=2, head_dim=128, q_lens=[70, 3], ctx_lens=[9050, 4100],
                          scale=1 / math.sqrt(128))
    _, out, ref = _run(c)
    assert_close(out, ref, dtype, c.name)


def test_prefill_many_sequences():
    """300 short sequences of mixed cost: the longest-first work order reads
    the lengths of sequences beyond those it keeps in registers."""
    rng = np.random.default_rng(35)
    q_lens = rng.integers(0, 6, 300)
    ctx = rng.integers(0, 200, 300)
    q_lens[[3, 150, 299]] = [40, 33, 70]
    ctx[[3, 150, 299]] = [700, 0, 260]
    c = make_prefill_case(name="many", seed=35, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                          head_dim=128, q_lens=q_lens, ctx_lens=ctx, scale=0.09)
    _, out, ref = _run(c)
    assert_close(out, ref, "bf16", c.name)


def test_prefill_block_permutation_invariance_bit_exact():
    """The same data under a new random placement of the physical blocks gives
    the same bits: the kernel's arithmetic depends on logical positions only."""
    from gpu_helpers import dev_bits
    c = make_prefill_case(name="perm", seed=36, dtype="bf16", num_q_heads=16, num_kv_heads=4,
                          head_dim=128, q_lens=[90, 5, 300], ctx_lens=[200, 0, 1100],
                          scale=0.088, extra_blocks=7)
    g = PrefillOnGPU(c)
    g.write()
    base = host_bits(g.prefill()).copy()
    kc, vc = host_bits(g.k_cache), host_bits(g.v_cache)
    perm = np.random.default_rng(37).permutation(c.num_blocks)
    kp, vp = np.empty_like(kc), np.empty_like(vc)
    kp[perm], vp[perm] = kc, vc
    tables = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    g.k_cache, g.v_cache = dev_bits(kp, c.dtype), dev_bits(vp, c.dtype)
    g.tables = dev_int(tables)
    g.out = torch.zeros_like(g.q)
    np.testing.assert_array_equal(base, host_bits(g.prefill()))


def test_prefill_deterministic_repeat():
    c = make_prefill_case(name="repeat", seed=38, dtype="f16", num_q_heads=32, num_kv_heads=8,
                          head_dim=128, q_lens=[257, 64, 3], ctx_lens=[700, 2000, 0], scale=0.088)
    g = PrefillOnGPU(c)
    g.write()
    first = host_bits(g.prefill()).copy()
    for _ in range(3):
        g.out = torch.zeros_like(g.q)
        np.testing.assert_array_equal(first, host_bits(g.prefill()))

