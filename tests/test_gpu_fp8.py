"""GPU parity of the FP8 (E4M3) KV cache against the float64 oracle: the
cache write bit-exact (codes and scales), decode within the 16-bit output
tolerance, and GPU-vs-GPU invariances.  Everything goes through the C ABI."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (TOL, Fp8DecodeOnGPU, Fp8PrefillOnGPU, assert_close, dev_bits, dev_int, host_bits, host_f64,
                         require_gpu)
from oracle_pins_fp8 import tie_rows_f16
from workloads import (decode_gqa_shared_prefix, decode_llama2_7b_layer, decode_long_context,
                       decode_tiny, make_decode_case, make_prefill_case, normal_bits,
                       prefill_chunked)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import paged_kv_cache_24_amd  # noqa: F401  (fails loudly without libpa.so)


def _codes(t):
    return t.cpu().numpy()


def _check_pools(g):
    kc, vc, ks, vs = g.oracle_pools()
    np.testing.assert_array_equal(_codes(g.k_cache), kc)
    np.testing.assert_array_equal(_codes(g.v_cache), vc)
    np.testing.assert_array_equal(g.k_scales.cpu().numpy(), ks)     # NaN where never written
    np.testing.assert_array_equal(g.v_scales.cpu().numpy(), vs)
    return kc, vc, ks, vs


def _check_fp8_case(c, partitions=(0,)):
    """FP8 cache write bit-exact; decode within tolerance for every partition
    length; the streaming hint changes no bit."""
    import paged_kv_cache_24_amd as pa
    g = Fp8DecodeOnGPU(c)
    g.write()
    torch.cuda.synchronize()
    kc, vc, ks, vs = _check_pools(g)
    ref = oracle.ref_decode_fp8(c.q, kc, vc, ks, vs, c.block_tables, c.seq_lens, c.scale, c.dtype)
    errs = {}
    for p in partitions:
        out = g.decode(partition_tokens=p)
        torch.cuda.synchronize()
        errs[p] = assert_close(host_f64(out), ref, c.dtype, f"{c.name} fp8 partition={p}")
        plain = host_bits(out).copy()
        streamed = host_bits(g.decode(partition_tokens=p, flags=pa.PA_DECODE_STREAM_KV))
        np.testing.assert_array_equal(plain, streamed)
    return errs


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_cache_write_bit_exact(dtype, d):
    """Random rows, all-zero rows, a row with a -0, padding slots; codes and
    scales must equal the oracle's bit for bit."""
    import paged_kv_cache_24_amd as pa
    rng = np.random.default_rng(200 + d)
    n, hkv, nb = 37, 3, 8
    key = normal_bits(rng, (n, hkv, d), dtype)
    value = normal_bits(rng, (n, hkv, d), dtype)
    key[5] = 0
    value[6, 1] = 0
    key[7, 2, 3] = 0x8000
    value[8] = (value[8].astype(np.uint32) | 0x8000).astype(np.uint16)   # all negative
    slots = rng.permutation(nb * 16)[:n].astype(np.int64)
    slots[[3, 11]] = -1
    codes0 = np.full((nb, 16, hkv, d), 0x7F, np.uint8)
    sc0 = np.full((nb, hkv, 16), np.nan, np.float32)
    kc, vc = torch.from_numpy(codes0).cuda(), torch.from_numpy(codes0).cuda()
    ks, vs = torch.from_numpy(sc0).cuda(), torch.from_numpy(sc0).cuda()
    pa.pa_reshape_and_cache_fp8(dev_bits(key, dtype), dev_bits(value, dtype), kc, vc, ks, vs,
                                dev_int(slots, torch.int64))
    want = oracle.ref_reshape_and_cache_fp8(key, value, codes0, codes0, sc0, sc0, slots, dtype)
    for got, exp in zip((kc, vc, ks, vs), want):
        np.testing.assert_array_equal(got.cpu().numpy(), exp)


def test_fp8_cache_write_float32_quotient_ties():
    """Rows whose float32 quotients x / s fall exactly on E4M3 ties: only a
    correctly rounded float32 division followed by ties-to-even matches."""
    import paged_kv_cache_24_amd as pa
    rows = tie_rows_f16()                              # [rows, 1, 16]
    d = 64
    key = np.zeros((rows.shape[0], 1, d), np.uint16)
    key[:, :, :16] = rows
    key[:, :, 16:32] = rows                            # the tie pattern twice per row
    slots = np.arange(rows.shape[0], dtype=np.int64)
    codes0 = np.zeros((1, 16, 1, d), np.uint8)
    sc0 = np.zeros((1, 1, 16), np.float32)
    kc, vc = torch.from_numpy(codes0).cuda(), torch.from_numpy(codes0).cuda()
    ks, vs = torch.from_numpy(sc0).cuda(), torch.from_numpy(sc0).cuda()
    pa.pa_reshape_and_cache_fp8(dev_bits(key, "f16"), dev_bits(key, "f16"), kc, vc, ks, vs,
                                dev_int(slots, torch.int64))
    want = oracle.ref_reshape_and_cache_fp8(key, key, codes0, codes0, sc0, sc0, slots, "f16")
    np.testing.assert_array_equal(kc.cpu().numpy(), want[0])
    np.testing.assert_array_equal(ks.cpu().numpy(), want[2])


def test_fp8_decode_tiny():
    _check_fp8_case(decode_tiny(), partitions=(0, 16, 32, 112, -1))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (6, 2), (8, 2), (16, 2), (16, 1), (48, 2),
                                    (71, 1)])
def test_fp8_decode_shapes(dtype, d, hq, hkv):
    lens = [0, 1, 2, 15, 16, 17, 31, 33, 64, 100, 257, 300]
    c = make_decode_case(name=f"fp8-{dtype}-{d}-{hq}-{hkv}", seed=300 + hq + d, dtype=dtype,
                         num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seq_lens=lens,
                         num_blocks=64, max_blocks_per_seq=20, scale=1 / math.sqrt(d),
                         write_last=True)
    _check_fp8_case(c, partitions=(0, 16, 48, 256, 320, -1))


def test_fp8_decode_llama_reduced():
    c = decode_llama2_7b_layer(batch=6, max_len=1024, num_heads=32)
    _check_fp8_case(c, partitions=(0, 256, 1024, -1))


def test_fp8_decode_gqa_shared_prefix_reduced():
    c = decode_gqa_shared_prefix(batch=32, max_len=2048, min_len=128, group=16, prefix=1024)
    _check_fp8_case(c, partitions=(0, 512, 2048, -1))


def test_fp8_decode_long_reduced():
    c = decode_long_context(batch=2, seq_len=8192, num_blocks=1100)
    _check_fp8_case(c, partitions=(0, 256, 2048, -1))


def test_fp8_wide_value_range():
    """Rows scaled by powers of two from 2^-12 to 2^8 (per token and head): the
    V scales span tiny to large, which the kernels must carry without losing
    the probabilities' precision (fp16, where a naive fold would underflow)."""
    for dtype, hq in (("f16", 8), ("bf16", 4), ("f16", 2)):
        c = make_decode_case(name=f"fp8-range-{dtype}", seed=41, dtype=dtype, num_q_heads=hq,
                             num_kv_heads=2, head_dim=128, seq_lens=[5, 70, 300, 33],
                             num_blocks=40, max_blocks_per_seq=20, scale=0.08, write_last=False)
        g = Fp8DecodeOnGPU(c)
        rng = np.random.default_rng(42)
        k = rng.integers(-12, 9, size=g.key_np.shape[:2])
        for arr in (g.key_np, g.value_np):
            x = oracle.bits_to_float64(arr, dtype) * np.ldexp(1.0, k)[..., None]
            if dtype == "f16":
                arr[:] = x.astype(np.float16).view(np.uint16)
            else:
                arr[:] = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        g.key = dev_bits(g.key_np, dtype)
        g.value = dev_bits(g.value_np, dtype)
        g.write()
        kc, vc, ks, vs = _check_pools(g)
        ref = oracle.ref_decode_fp8(c.q, kc, vc, ks, vs, c.block_tables, c.seq_lens, c.scale, dtype)
        # the output is a convex combination of v rows: measure its error against
        # the largest |v| the sequence's kv head holds, with the usual tolerances
        vmax = np.zeros((c.num_seqs, c.num_q_heads, 1))
        for b in range(c.num_seqs):
            n = int(c.seq_lens[b])
            v = oracle.dequantize_e4m3_rows(oracle.gather_tokens(vc, c.block_tables[b], n),
                                            oracle.gather_scales(vs, c.block_tables[b], n))
            vmax[b, :, 0] = np.abs(v).max(axis=(0, 2))[np.arange(c.num_q_heads) // (hq // 2)]
        for p in (0, 64):
            out = g.decode(partition_tokens=p)
            torch.cuda.synchronize()
            rel = float((np.abs(host_f64(out) - ref) / vmax).max())
            assert rel <= TOL[dtype], (dtype, p, rel)


def test_fp8_block_permutation_invariance_bit_exact():
    c = decode_gqa_shared_prefix(batch=16, max_len=1024, min_len=16, group=4, prefix=256)
    g = Fp8DecodeOnGPU(c)
    g.write()
    base = host_bits(g.decode()).copy()
    perm = torch.from_numpy(np.random.default_rng(9).permutation(c.num_blocks)).cuda()
    for name in ("k_cache", "v_cache", "k_scales", "v_scales"):
        t = getattr(g, name)
        moved = torch.empty_like(t)
        moved[perm] = t
        setattr(g, name, moved)
    tables = torch.where(g.tables >= 0, perm[g.tables.clamp(min=0).long()].int(), g.tables)
    g.tables = tables.contiguous()
    np.testing.assert_array_equal(host_bits(g.decode()), base)


def test_fp8_copy_blocks_then_decode():
    """Copy-on-write on an FP8 cache: copy blocks (codes and scales), point one
    sequence at the copies; its output must not change by a bit."""
    import paged_kv_cache_24_amd as pa
    c = make_decode_case(name="fp8-cow", seed=77, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                         head_dim=128, seq_lens=[40, 70], num_blocks=16, max_blocks_per_seq=5,
                         scale=0.09, write_last=False)
    g = Fp8DecodeOnGPU(c)
    g.write()
    base = host_bits(g.decode()).copy()
    used = set(int(x) for x in c.block_tables[c.block_tables >= 0])
    spare = [b for b in range(16) if b not in used]
    row = [int(x) for x in c.block_tables[1] if x >= 0]
    pairs = np.array([[s, spare[i]] for i, s in enumerate(row)], np.int64)
    pa.pa_copy_blocks_fp8(g.k_cache, g.v_cache, g.k_scales, g.v_scales, dev_int(pairs, torch.int64))
    torch.cuda.synchronize()
    for t in (g.k_cache, g.v_cache, g.k_scales, g.v_scales):
        h = t.cpu().numpy()
        for s, dst in pairs:
            np.testing.assert_array_equal(h[dst], h[s])
    tables = c.block_tables.copy()
    tables[1, :len(row)] = pairs[:, 1]
    g.tables = dev_int(tables)
    np.testing.assert_array_equal(host_bits(g.decode()), base)


def test_fp8_empty_and_zero_lengths():
    c = make_decode_case(name="fp8-zero", seed=5, dtype="f16", num_q_heads=4, num_kv_heads=4,
                         head_dim=64, seq_lens=[0, 3, 0], num_blocks=4, max_blocks_per_seq=2,
                         scale=0.125, write_last=False)
    g = Fp8DecodeOnGPU(c)
    g.write()
    out = host_f64(g.decode())
    assert (out[0] == 0).all() and (out[2] == 0).all() and np.isfinite(out).all()


def _check_fp8_prefill(c):
    g = Fp8PrefillOnGPU(c)
    g.write()
    torch.cuda.synchronize()
    kc, vc, ks, vs = g.oracle_pools()
    np.testing.assert_array_equal(g.k_cache.cpu().numpy(), kc)
    np.testing.assert_array_equal(g.v_scales.cpu().numpy(), vs)
    out = host_f64(g.prefill())
    ref = oracle.ref_prefill_paged_fp8(c.q, kc, vc, ks, vs, c.block_tables, c.ctx_lens,
                                       c.query_start_loc, c.scale, c.dtype)
    return assert_close(out, ref, c.dtype, c.name + " fp8")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (8, 2), (16, 2), (12, 4), (10, 2), (12, 2),
                                    (14, 2), (16, 1)])
def test_fp8_prefill_shapes(dtype, hq, hkv, d):
    q_lens = [0, 1, 17, 64, 130, 5, 33]
    ctx = [3, 0, 40, 0, 100, 16, 250]
    seed = 400 + hq if d == 128 else 500 + hq
    c = make_prefill_case(name=f"prefill-{dtype}-{hq}-{hkv}-d{d}", seed=seed, dtype=dtype,
                          num_q_heads=hq, num_kv_heads=hkv, head_dim=d, q_lens=q_lens,
                          ctx_lens=ctx, scale=1 / math.sqrt(d), extra_blocks=5)
    _check_fp8_prefill(c)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(48, 2), (64, 2), (128, 1)])
def test_fp8_prefill_large_groups(hq, hkv, d):
    """24, 32 and 128 q heads per kv head over the FP8 cache: a workgroup holds
    few positions (idle rows when the group does not divide it)."""
    c = make_prefill_case(name=f"fp8-prefill-group-{hq // hkv}-d{d}", seed=93 + hq + d,
                          dtype="bf16", num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                          q_lens=[9, 0, 4, 1, 23], ctx_lens=[30, 5, 0, 70, 2],
                          scale=1 / math.sqrt(d), extra_blocks=2)
    _check_fp8_prefill(c)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp8_prefill_long_context(dtype):
    """~9000 cached keys over the FP8 cache: many key tiles per workgroup."""
    c = make_prefill_case(name=f"fp8-long-{dtype}", seed=36, dtype=dtype, num_q_heads=8,
                          num_kv_heads=2, head_dim=128, q_lens=[70, 3], ctx_lens=[9050, 4100],
                          scale=1 / math.sqrt(128))
    _check_fp8_prefill(c)


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_prefill_wide_value_range(d):
    """The prefill counterpart of the decode range test: k and v rows scaled by
    powers of two from 2^-12 to 2^8 per token and head, so that the scales'
    exponents and mantissa factors span a wide range on every key tile."""
    for dtype, hq in (("f16", 8), ("bf16", 4), ("f16", 2)):
        c = make_prefill_case(name=f"fp8-prefill-range-{dtype}-{hq}-d{d}", seed=43 + hq + d,
                              dtype=dtype, num_q_heads=hq, num_kv_heads=2, head_dim=d,
                              q_lens=[5, 70, 130, 33], ctx_lens=[0, 40, 170, 3], scale=0.08)
        g = Fp8PrefillOnGPU(c)
        rng = np.random.default_rng(44)
        k = rng.integers(-12, 9, size=g.key_np.shape[:2])
        for arr in (g.key_np, g.value_np):
            x = oracle.bits_to_float64(arr, dtype) * np.ldexp(1.0, k)[..., None]
            if dtype == "f16":
                arr[:] = x.astype(np.float16).view(np.uint16)
            else:
                arr[:] = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        g.key = dev_bits(g.key_np, dtype)
        g.value = dev_bits(g.value_np, dtype)
        g.write()
        kc, vc, ks, vs = _check_pools(g)
        ref = oracle.ref_prefill_paged_fp8(c.q, kc, vc, ks, vs, c.block_tables, c.ctx_lens,
                                           c.query_start_loc, c.scale, dtype)
        out = host_f64(g.prefill())
        # a convex combination of v rows: the error is measured against the
        # largest |v| of the sequence's kv head, with the usual tolerances
        vmax = np.ones_like(ref[..., :1])
        for b in range(c.num_seqs):
            lo, hi = int(c.query_start_loc[b]), int(c.query_start_loc[b + 1])
            n = int(c.ctx_lens[b] + c.q_lens[b])
            v = oracle.dequantize_e4m3_rows(oracle.gather_tokens(vc, c.block_tables[b], n),
                                            oracle.gather_scales(vs, c.block_tables[b], n))
            vmax[lo:hi, :, 0] = np.abs(v).max(axis=(0, 2))[np.arange(hq) // (hq // 2)]
        rel = float((np.abs(out - ref) / vmax).max())
        assert rel <= TOL[dtype], (dtype, hq, d, rel)


def test_fp8_prefill_chunked_reduced():
    _check_fp8_prefill(prefill_chunked(batch=4, new_tokens=600, max_ctx=700))


def test_fp8_prefill_row_matches_fp8_decode():
    """The last row of a chunk and a decode of the same position over the same
    FP8 cache attend to the same keys: they must agree to the tolerance."""
    import paged_kv_cache_24_amd as pa
    c = make_prefill_case(name="fp8-row", seed=47, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                          head_dim=128, q_lens=[37, 70], ctx_lens=[200, 3], scale=0.09)
    g = Fp8PrefillOnGPU(c)
    g.write()
    out = host_f64(g.prefill())
    for b in range(2):
        r = int(c.query_start_loc[b + 1]) - 1
        n = int(c.ctx_lens[b] + c.q_lens[b])
        dec = torch.empty((1, 8, 128), dtype=torch.bfloat16, device="cuda")
        pa.pa_decode_fp8(dec, g.q[r:r + 1].contiguous(), g.k_cache, g.v_cache, g.k_scales, g.v_scales,
                         g.tables[b:b + 1].contiguous(), dev_int(np.array([n], np.int32)), c.scale)
        assert float(np.abs(host_f64(dec)[0] - out[r]).max()) <= 1e-2
