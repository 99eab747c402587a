"""GPU parity of multi-query decode (draft-token verification) against the
float64 oracle, and its consistency with single-query decode.  Everything
goes through the C ABI."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (DecodeOnGPU, assert_close, dev_bits, dev_int, host_bits, host_f64,
                         require_gpu)
from workloads import decode_llama2_7b_layer, make_decode_case, normal_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import paged_kv_cache_24_amd  # noqa: F401  (fails loudly without libpa.so)


def _multi(g, qm, part=0, flags=0):
    import paged_kv_cache_24_amd as pa
    out = torch.empty_like(qm)
    pa.pa_decode_multi(out, qm, g.k_cache, g.v_cache, g.tables, g.lens, g.case.scale, part,
                       flags=flags)
    torch.cuda.synchronize()
    return out


def _check(c, nq, partitions=(0,), seed=1):
    import paged_kv_cache_24_amd as pa
    g = DecodeOnGPU(c)
    g.write()
    kc, vc = oracle.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    q = normal_bits(np.random.default_rng(seed), (c.num_seqs, nq, c.num_q_heads, c.head_dim), c.dtype)
    qm = dev_bits(q, c.dtype)
    ref = oracle.ref_decode_multi(q, kc, vc, c.block_tables, c.seq_lens, c.scale, c.dtype)
    for p in partitions:
        out = _multi(g, qm, p)
        assert_close(host_f64(out), ref, c.dtype, f"{c.name} Q={nq} partition={p}")
        streamed = _multi(g, qm, p, pa.PA_DECODE_STREAM_KV)
        np.testing.assert_array_equal(host_bits(out), host_bits(streamed))
    return g, q, qm


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (16, 2), (32, 4)])
@pytest.mark.parametrize("nq", [2, 4, 7])
def test_multi_shapes(dtype, d, hq, hkv, nq):
    lens = [0, 1, 2, 5, 15, 16, 17, 33, 100, 257, 300]
    c = make_decode_case(name=f"multi-{dtype}-{d}-{hq}-{hkv}", seed=500 + hq + d + nq, dtype=dtype,
                         num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seq_lens=lens,
                         num_blocks=64, max_blocks_per_seq=20, scale=1 / math.sqrt(d),
                         write_last=True)
    _check(c, nq, partitions=(0, 16, 48, 320))


def test_multi_llama_reduced():
    c = decode_llama2_7b_layer(batch=6, max_len=1024, num_heads=32)
    _check(c, 4, partitions=(0, 256, 1024))


def test_multi_single_query_is_decode_bit_exact():
    """q_per_seq = 1 runs the plain decode kernels: bit-identical to pa_decode."""
    c = make_decode_case(name="multi-one", seed=61, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                         head_dim=128, seq_lens=[3, 40, 129, 600], num_blocks=64,
                         max_blocks_per_seq=40, scale=0.08, write_last=True)
    g = DecodeOnGPU(c)
    g.write()
    for p in (0, 64):
        single = host_bits(g.decode(partition_tokens=p)).copy()
        multi = host_bits(_multi(g, g.q[:, None].contiguous(), p))[:, 0]
        np.testing.assert_array_equal(multi, single)


def test_multi_rows_match_rolled_back_decodes():
    """Row j of a verification pass and a plain decode of the same query with
    seq_len n - Q + j + 1 (the sequence after rejecting the later drafts)."""
    nq = 5
    c = make_decode_case(name="multi-roll", seed=62, dtype="f16", num_q_heads=32, num_kv_heads=32,
                         head_dim=128, seq_lens=[7, 90, 513], num_blocks=60, max_blocks_per_seq=40,
                         scale=0.088, write_last=False)
    g, q, qm = _check(c, nq)
    out = host_f64(_multi(g, qm))
    import paged_kv_cache_24_amd as pa
    for j in range(nq):
        lens = np.maximum(c.seq_lens - nq + j + 1, 0).astype(np.int32)
        dec = torch.empty_like(g.q)
        pa.pa_decode(dec, qm[:, j].contiguous(), g.k_cache, g.v_cache, g.tables, dev_int(lens), c.scale)
        torch.cuda.synchronize()
        assert float(np.abs(host_f64(dec) - out[:, j]).max()) <= 2e-3


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_multi_balanced_split(dtype):
    """Several queries on matrix cores in the balanced split (partition 0 takes it
    when its partial states, (16 + 96 stretches) x 32 units x 4 columns, fit the
    documented workspace, 64 x 32 x 8 states of 512-token partitions: 32 heads,
    4096-token tables): against the oracle, beside fixed 1024-token partitions."""
    lens = [4096, 1, 2, 3, 4, 5, 17, 1000, 2500, 16, 3333, 64, 0, 4095, 129, 700]
    c = make_decode_case(name=f"multi-balanced-{dtype}", seed=531, dtype=dtype, num_q_heads=32,
                         num_kv_heads=32, head_dim=128, seq_lens=lens,
                         num_blocks=sum((n + 15) // 16 for n in lens) + 4, max_blocks_per_seq=256,
                         scale=1 / math.sqrt(128), write_last=True)
    _check(c, 4, partitions=(0, 1024))


def test_multi_balanced_split_head_chunks():
    """32 (query, head) columns per kv head (8 q heads x 4 queries): two column
    chunks per kv head in the balanced split (128 sequences, 2048-token tables,
    so that its states fit the documented workspace)."""
    rng = np.random.default_rng(532)
    lens = rng.integers(0, 2049, 128)
    lens[:6] = [0, 1, 2, 3, 4, 2048]
    c = make_decode_case(name="multi-balanced-chunks", seed=533, dtype="bf16", num_q_heads=16,
                         num_kv_heads=2, head_dim=128, seq_lens=lens,
                         num_blocks=int(sum((n + 15) // 16 for n in lens)) + 4, max_blocks_per_seq=128,
                         scale=1 / math.sqrt(128), write_last=True)
    _check(c, 4, partitions=(0,))
