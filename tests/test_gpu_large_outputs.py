"""Large bf16 outputs (|out| >= 4) through the matrix-core and FP8 paths.

Where |out| >= 4 a bf16 output is spaced 2^-5 apart or more, so even a
correctly rounded result can miss the 1e-2 tolerance.  These cases (short
contexts, V scaled by 16, q and k N(0, 1)) are checked element by element
against a bound derived from each path's arithmetic instead, and the worst
error is printed in ulps of bf16 (spacings of the output type at the
oracle's value):

    |got - ref| <= spacing(ref)/2  +  2u/(1-2u) * sum_j w_j |v_j - ref|
                                   +  eps * sum_j w_j |v_j|

* spacing/2: the final round to bf16.
* 2u term: the matrix-core paths (GQA decode and prefill, 16-bit and FP8)
  round each weight to bf16 before the PV product (relative error <= u =
  2^-8) and their row sum adds the probabilities those rounded weights stand
  for (over FP8 the weight is p times the mantissa factor f of the key's v
  scale, and the sum adds weight / f), so the weights that multiply V still
  sum to one; a perturbation delta_j of each weight moves the output by
  sum_j w_j (delta_j - mean delta)(v_j - ref).  With a row sum of unrounded p
  the error would grow with |v| instead of with the spread of v around the
  output.  The vector-ALU paths keep p in float32: u = 0.
* eps = 2^-13: float32 accumulation in the scores (head_dim 128 products),
  the sums and the division, bounded for these sizes.

The two weighted sums are the oracle's own attention applied to |V - ref|
and |V| (gpu_helpers.weighted_sums).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (EPS32, TORCH_DTYPE, DecodeOnGPU, PrefillOnGPU, Fp8DecodeOnGPU,
                         Fp8PrefillOnGPU, host_f64, require_gpu, ulps, weighted_sums)
from workloads import make_decode_case, make_prefill_case

pytestmark = pytest.mark.gpu

U_BF16 = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import paged_kv_cache_24_amd  # noqa: F401


def _scaled_bits(bits: np.ndarray, dtype: str, factor: float) -> np.ndarray:
    """16-bit patterns times a power of two (exact; NaN stays NaN)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH_DTYPE[dtype])
    return (t * factor).view(torch.int16).numpy().view(np.uint16)


def _check(got, ref, dev, mag, u, what):
    spacing = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    allowed = 0.5 * spacing + 2 * u / (1 - 2 * u) * dev + EPS32 * mag
    err = np.abs(got - ref)
    big = np.abs(ref) >= 4
    assert big.sum() > 100, "the case must really have outputs of magnitude 4 or more"
    ul = ulps(got, ref, "bf16")
    print(f"{what}: {int(big.sum())} outputs with |ref| >= 4, worst {ul[big].max():.3f} ulps "
          f"(bound there up to {(allowed / spacing)[big].max():.3f}); worst error/bound over all "
          f"outputs {(err / allowed).max():.3f}")
    i = np.unravel_index(int(np.argmax(err / allowed)), err.shape)
    assert (err <= allowed).all(), (f"{what}: error {err[i]:.4e} > bound {allowed[i]:.4e} at "
                                    f"{tuple(int(x) for x in i)} (ref {ref[i]:.4f})")


def _decode_case(hq, hkv, d, seed):
    c = make_decode_case(name=f"large-{hq}-{hkv}-{d}", seed=seed, dtype="bf16", num_q_heads=hq,
                         num_kv_heads=hkv, head_dim=d, seq_lens=[1, 2, 3, 2, 5, 3, 40, 4],
                         num_blocks=16, max_blocks_per_seq=3, scale=0.05, write_last=True)
    c.v_cache[:] = _scaled_bits(c.v_cache, "bf16", 16.0)
    c.value[:] = _scaled_bits(c.value, "bf16", 16.0)
    return c


@pytest.mark.parametrize("hq,hkv", [(16, 2), (8, 2)])
def test_gqa_decode_large_outputs(hq, hkv):
    """Matrix-core GQA decode (16-bit cache), split and unsplit."""
    c = _decode_case(hq, hkv, 128, seed=31 + hq)
    g = DecodeOnGPU(c)
    g.write()
    kc, vc = oracle.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    ref = oracle.ref_decode(c.q, kc, vc, c.block_tables, c.seq_lens, c.scale, "bf16")
    dev, mag = np.zeros_like(ref), np.zeros_like(ref)
    for b in range(c.num_seqs):
        n = int(c.seq_lens[b])
        k64 = oracle.bits_to_float64(oracle.gather_tokens(kc, c.block_tables[b], n), "bf16")
        v64 = oracle.bits_to_float64(oracle.gather_tokens(vc, c.block_tables[b], n), "bf16")
        q64 = oracle.bits_to_float64(c.q[b], "bf16")[None]
        dv, mg = weighted_sums(q64, k64, v64, np.array([n - 1]), c.scale, ref[b][None])
        dev[b], mag[b] = dv[0], mg[0]
    for part in (0, 16):
        got = host_f64(g.decode(partition_tokens=part))
        _check(got, ref, dev, mag, U_BF16, f"GQA decode {hq}/{hkv} partition {part}")


@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (4, 1, 128), (8, 2, 64)])
def test_prefill_large_outputs(hq, hkv, d):
    """16-bit prefill on matrix cores: head_dim 128 (32x32x16 kernel) and 64."""
    c = make_prefill_case(name=f"large-prefill-{hq}-{hkv}-{d}", seed=35 + d, dtype="bf16",
                          num_q_heads=hq, num_kv_heads=hkv, head_dim=d, q_lens=[6, 3, 20, 9],
                          ctx_lens=[0, 1, 2, 0], scale=0.05)
    c.v_cache[:] = _scaled_bits(c.v_cache, "bf16", 16.0)
    c.value[:] = _scaled_bits(c.value, "bf16", 16.0)
    g = PrefillOnGPU(c)
    g.write()
    got = host_f64(g.prefill())
    kc, vc = oracle.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    ref = oracle.ref_prefill_paged(c.q, kc, vc, c.block_tables, c.ctx_lens, c.query_start_loc,
                                   c.scale, "bf16")
    dev, mag = np.zeros_like(ref), np.zeros_like(ref)
    for b in range(c.num_seqs):
        lo, L, ctx = int(c.query_start_loc[b]), int(c.q_lens[b]), int(c.ctx_lens[b])
        n = ctx + L
        k64 = oracle.bits_to_float64(oracle.gather_tokens(kc, c.block_tables[b], n), "bf16")
        v64 = oracle.bits_to_float64(oracle.gather_tokens(vc, c.block_tables[b], n), "bf16")
        q64 = oracle.bits_to_float64(c.q[lo:lo + L], "bf16")
        dev[lo:lo + L], mag[lo:lo + L] = weighted_sums(q64, k64, v64, ctx + np.arange(L), c.scale,
                                                        ref[lo:lo + L])
    _check(got, ref, dev, mag, U_BF16, f"prefill {hq}/{hkv} D={d}")


def _fp8_tokens(codes, scales, table_row, n):
    return oracle.dequantize_e4m3_rows(oracle.gather_tokens(codes, table_row, n),
                                       oracle.gather_scales(scales, table_row, n))


@pytest.mark.parametrize("hq,hkv,u", [(16, 2, U_BF16), (4, 4, 0.0)])
def test_fp8_decode_large_outputs(hq, hkv, u):
    """FP8 decode: the matrix-core GQA kernel (16/2) and the vector kernel (4/4)."""
    c = _decode_case(hq, hkv, 128, seed=51 + hq)
    g = Fp8DecodeOnGPU(c)
    g.write()
    kc, vc, ks, vs = g.oracle_pools()
    ref = oracle.ref_decode_fp8(c.q, kc, vc, ks, vs, c.block_tables, c.seq_lens, c.scale, "bf16")
    dev, mag = np.zeros_like(ref), np.zeros_like(ref)
    for b in range(c.num_seqs):
        n = int(c.seq_lens[b])
        k64 = _fp8_tokens(kc, ks, c.block_tables[b], n)
        v64 = _fp8_tokens(vc, vs, c.block_tables[b], n)
        q64 = oracle.bits_to_float64(c.q[b], "bf16")[None]
        dv, mg = weighted_sums(q64, k64, v64, np.array([n - 1]), c.scale, ref[b][None])
        dev[b], mag[b] = dv[0], mg[0]
    for part in (0, 16):
        got = host_f64(g.decode(partition_tokens=part))
        _check(got, ref, dev, mag, u, f"FP8 decode {hq}/{hkv} partition {part}")


def test_fp8_prefill_large_outputs():
    c = make_prefill_case(name="large-prefill-fp8", seed=57, dtype="bf16", num_q_heads=8,
                          num_kv_heads=2, head_dim=128, q_lens=[6, 3, 20, 9], ctx_lens=[0, 1, 2, 0],
                          scale=0.05)
    c.v_cache[:] = _scaled_bits(c.v_cache, "bf16", 16.0)
    c.value[:] = _scaled_bits(c.value, "bf16", 16.0)
    g = Fp8PrefillOnGPU(c)
    g.write()
    got = host_f64(g.prefill())
    kc, vc, ks, vs = g.oracle_pools()
    ref = oracle.ref_prefill_paged_fp8(c.q, kc, vc, ks, vs, c.block_tables, c.ctx_lens,
                                       c.query_start_loc, c.scale, "bf16")
    dev, mag = np.zeros_like(ref), np.zeros_like(ref)
    for b in range(c.num_seqs):
        lo, L, ctx = int(c.query_start_loc[b]), int(c.q_lens[b]), int(c.ctx_lens[b])
        n = ctx + L
        k64 = _fp8_tokens(kc, ks, c.block_tables[b], n)
        v64 = _fp8_tokens(vc, vs, c.block_tables[b], n)
        q64 = oracle.bits_to_float64(c.q[lo:lo + L], "bf16")
        dev[lo:lo + L], mag[lo:lo + L] = weighted_sums(q64, k64, v64, ctx + np.arange(L), c.scale,
                                                        ref[lo:lo + L])
    _check(got, ref, dev, mag, U_BF16, "FP8 prefill 8/2")
