"""GPU parity with 32-token cache blocks.

Each workload is drawn twice from one seed: once in 16-token blocks and once
in 32-token blocks (the generators draw the same tokens for either layout,
only the pool and the tables differ).  With 32-token blocks the cache write
and the block copy must match the oracle bit for bit, and decode / prefill
must be within tolerance of the oracle.  The kernels walk a 32-token block as
two 16-token halves in the same order as two 16-token blocks, so the output
must also be bit-identical to the 16-token layout's.  Everything goes through
the C ABI."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (DecodeOnGPU, PrefillOnGPU, assert_close, dev_bits, dev_int, host_bits,
                         host_f64, require_gpu)
from workloads import (decode_gqa_shared_prefix, decode_llama2_7b_layer, make_decode_case,
                       make_prefill_case, normal_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import paged_kv_cache_24_amd  # noqa: F401  (fails loudly without libpa.so)


def _pair(make, **kw):
    """The same workload in 16- and 32-token blocks."""
    return make(block_size=16, **kw), make(block_size=32, **kw)


def _written(c):
    return oracle.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)


LENS = [1, 15, 16, 17, 31, 32, 33, 64, 100, 257, 511, 0]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (8, 2), (16, 2), (48, 2)])
def test_block32_decode(dtype, d, hq, hkv):
    """Vector path (group <= 2), matrix-core path (group 3..16 at head_dim 128)
    and head chunks (group 24); partitions of 16 tokens split every 32-token
    block between two partitions."""
    import paged_kv_cache_24_amd as pa

    def make(block_size):
        return make_decode_case(name=f"bs{block_size}-{dtype}-{d}-{hq}-{hkv}", seed=900 + hq + d,
                                dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                seq_lens=LENS, num_blocks=2048 // block_size + 3,
                                max_blocks_per_seq=512 // block_size, scale=1 / math.sqrt(d),
                                write_last=True, block_size=block_size)
    c16, c32 = _pair(make)
    g16, g32 = DecodeOnGPU(c16), DecodeOnGPU(c32)
    g16.write()
    g32.write()
    kc, vc = _written(c32)
    np.testing.assert_array_equal(host_bits(g32.k_cache), kc)   # the cache write is a bit copy
    np.testing.assert_array_equal(host_bits(g32.v_cache), vc)
    ref = oracle.ref_decode(c32.q, kc, vc, c32.block_tables, c32.seq_lens, c32.scale, dtype)
    for p in (0, 16, 48, 256):
        out32 = host_bits(g32.decode(partition_tokens=p)).copy()
        out16 = host_bits(g16.decode(partition_tokens=p)).copy()
        torch.cuda.synchronize()
        assert_close(host_f64(g32.out), ref, dtype, f"{c32.name} partition={p}")
        np.testing.assert_array_equal(out32, out16)
        streamed = host_bits(g32.decode(partition_tokens=p, flags=pa.PA_DECODE_STREAM_KV))
        np.testing.assert_array_equal(streamed, out32)


@pytest.mark.parametrize("nq", [2, 4])
@pytest.mark.parametrize("hq,hkv", [(32, 32), (32, 8)])
def test_block32_decode_multi(nq, hq, hkv):
    import paged_kv_cache_24_amd as pa

    def make(block_size):
        return make_decode_case(name=f"multi-bs{block_size}-{hq}-{hkv}", seed=950 + nq + hkv,
                                dtype="bf16", num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                                seq_lens=LENS, num_blocks=2048 // block_size + 1,
                                max_blocks_per_seq=512 // block_size, scale=1 / math.sqrt(128),
                                write_last=True, block_size=block_size)
    c16, c32 = _pair(make)
    g16, g32 = DecodeOnGPU(c16), DecodeOnGPU(c32)
    g16.write()
    g32.write()
    kc, vc = _written(c32)
    q = normal_bits(np.random.default_rng(nq), (c32.num_seqs, nq, hq, 128), "bf16")
    qm = dev_bits(q, "bf16")
    ref = oracle.ref_decode_multi(q, kc, vc, c32.block_tables, c32.seq_lens, c32.scale, "bf16")
    for p in (0, 16, 96):
        outs = []
        for g in (g32, g16):
            out = torch.empty_like(qm)
            pa.pa_decode_multi(out, qm, g.k_cache, g.v_cache, g.tables, g.lens, g.case.scale, p)
            outs.append(out)
        torch.cuda.synchronize()
        assert_close(host_f64(outs[0]), ref, "bf16", f"{c32.name} Q={nq} partition={p}")
        np.testing.assert_array_equal(host_bits(outs[0]), host_bits(outs[1]))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8), (16, 2)])
def test_block32_prefill(dtype, d, hq, hkv):
    """Both prefill kernels (head_dim 128 and 64) over 32-token blocks: ragged
    chunks, contexts that end inside either half of a block, an empty chunk."""
    q_lens = [0, 1, 17, 64, 130, 5, 33, 200]
    ctx = [3, 0, 40, 16, 100, 31, 250, 47]

    def make(block_size):
        return make_prefill_case(name=f"prefill-bs{block_size}-{dtype}-{hq}-{hkv}-d{d}",
                                 seed=970 + hq + d, dtype=dtype, num_q_heads=hq,
                                 num_kv_heads=hkv, head_dim=d, q_lens=q_lens, ctx_lens=ctx,
                                 scale=1 / math.sqrt(d), extra_blocks=3, block_size=block_size)
    c16, c32 = _pair(make)
    g16, g32 = PrefillOnGPU(c16), PrefillOnGPU(c32)
    g16.write()
    g32.write()
    kc, vc = _written(c32)
    np.testing.assert_array_equal(host_bits(g32.k_cache), kc)
    np.testing.assert_array_equal(host_bits(g32.v_cache), vc)
    out32 = host_bits(g32.prefill()).copy()
    out16 = host_bits(g16.prefill()).copy()
    ref = oracle.ref_prefill_paged(c32.q, kc, vc, c32.block_tables, c32.ctx_lens,
                                   c32.query_start_loc, c32.scale, dtype)
    assert_close(host_f64(g32.out), ref, dtype, c32.name)
    np.testing.assert_array_equal(out32, out16)


def test_block32_shared_prefix():
    """Groups of 8 sequences share a 512-token prefix (16 blocks of 32 tokens)."""
    c16, c32 = _pair(decode_gqa_shared_prefix, seed=33, batch=24, max_len=2048, min_len=64, group=8,
                     prefix=512)
    g16, g32 = DecodeOnGPU(c16), DecodeOnGPU(c32)
    out32 = host_bits(g32.decode()).copy()
    out16 = host_bits(g16.decode()).copy()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out32, out16)
    ref = oracle.ref_decode(c32.q, c32.k_cache, c32.v_cache, c32.block_tables, c32.seq_lens,
                            c32.scale, "bf16")
    assert_close(host_f64(g32.out), ref, "bf16", c32.name)


def test_block32_llama_layer_partial():
    """The LLaMA-2-7B-shaped layer (32 heads, head_dim 128, fp16, lengths up to
    4096) for 8 sequences in 32-token blocks; oracle on every sequence."""
    c16, c32 = _pair(decode_llama2_7b_layer, seed=34, batch=8)
    g16, g32 = DecodeOnGPU(c16), DecodeOnGPU(c32)
    g16.write()
    g32.write()
    out32 = host_bits(g32.decode()).copy()
    out16 = host_bits(g16.decode()).copy()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out32, out16)
    kc, vc = _written(c32)
    ref = oracle.ref_decode(c32.q, kc, vc, c32.block_tables, c32.seq_lens, c32.scale, "f16")
    assert_close(host_f64(g32.out), ref, "f16", c32.name)


def test_block32_copy_blocks():
    """Block copy of whole 32-token blocks against the oracle, whole pools."""
    import paged_kv_cache_24_amd as pa
    rng = np.random.default_rng(35)
    for dtype, hkv, d in (("bf16", 8, 128), ("f16", 4, 64)):
        nb = 30
        kc = normal_bits(rng, (nb, 32, hkv, d), dtype)
        vc = normal_bits(rng, (nb, 32, hkv, d), dtype)
        perm = rng.permutation(nb)
        pairs = np.stack([perm[:10], perm[10:20]], axis=1).astype(np.int64)
        pairs = np.concatenate([pairs, [[-1, 5], [perm[25], nb]]]).astype(np.int64)
        gk, gv = dev_bits(kc, dtype), dev_bits(vc, dtype)
        pa.pa_copy_blocks(gk, gv, dev_int(pairs, torch.int64))
        ok = pairs[(pairs[:, 0] >= 0) & (pairs[:, 1] >= 0) & (pairs[:, 1] < nb)]
        rk, rv = oracle.ref_copy_blocks(kc, vc, ok)
        np.testing.assert_array_equal(host_bits(gk), rk)
        np.testing.assert_array_equal(host_bits(gv), rv)


def test_block32_two_phase_decode_equals_one_call():
    """pa_decode_partitions then pa_decode_merge (both told block_size 32) give
    exactly the output of pa_decode."""
    import paged_kv_cache_24_amd as pa
    c = make_decode_case(name="two-phase-bs32", seed=980, dtype="bf16", num_q_heads=16,
                         num_kv_heads=2, head_dim=128, seq_lens=LENS, num_blocks=70,
                         max_blocks_per_seq=16, scale=1 / math.sqrt(128), write_last=True,
                         block_size=32)
    g = DecodeOnGPU(c)
    g.write()
    for p in (0, 64):
        one = host_bits(g.decode(partition_tokens=p)).copy()
        need = pa.pa_decode_workspace_size(c.num_seqs, 16, 2, 128, 32, 16, p)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(g.q)
        pa.pa_decode_partitions(out, g.q, g.k_cache, g.v_cache, g.tables, g.lens, c.scale, ws, p)
        pa.pa_decode_merge(out, g.lens, 2, 16, ws, p, block_size=32)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(out), one)
