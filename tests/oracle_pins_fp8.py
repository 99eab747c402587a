"""Checks that pin the FP8 (E4M3) part of the oracle to facts fixed outside it.

Each ``pin_*`` takes the FP8 oracle module (``oracle.kv_fp8`` or a mutated
copy) and raises ``AssertionError`` when it disagrees with:

* the E4M3 format itself: closed-form values of its codes, torch's
  ``float8_e4m3fn`` conversions on the CPU (an independent implementation of
  the same encoding), and brute-force nearest-value search;
* invariants of per-row scaling (the largest element lands on 448, the error
  bound of round-to-nearest, sign symmetry, power-of-two scaling);
* the unquantised oracle, on inputs whose quantisation is lossless: then the
  FP8 cache must give exactly the same attention as the 16-bit one.

``test_oracle_pins_fp8.py`` runs them on the real module and
``test_oracle_fp8_mutants.py`` plants mistakes and checks some pin fails.
"""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle.paged_attention as pa
from workloads import make_decode_case, make_prefill_case, normal_bits

_ALL_CODES = np.arange(256, dtype=np.uint8)


def _torch_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _finite_table():
    """(codes, values) of the 254 finite non-NaN codes, by closed form."""
    vals, codes = [], []
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        vals.append(-v if s else v)
        codes.append(c)
    return np.array(codes), np.array(vals)


# ------------------------------------------------------------------ the format

def pin_e4m3_closed_form_codes(o):
    got = o.e4m3_to_float64(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x7E, 0xC0, 0x80, 0x7F, 0xFF],
                                     np.uint8))
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.5, 448.0, -2.0, -0.0]
    np.testing.assert_array_equal(got[:9], want)
    assert np.signbit(got[8]) and not np.signbit(got[0])
    assert np.isnan(got[9]) and np.isnan(got[10])
    assert o.E4M3_MAX == 448.0


def pin_e4m3_decode_matches_torch(o):
    np.testing.assert_array_equal(o.e4m3_to_float64(_ALL_CODES), _torch_decode(_ALL_CODES))


def pin_e4m3_encode_round_trip_and_saturation(o):
    codes, vals = _finite_table()
    np.testing.assert_array_equal(o.float_to_e4m3(vals), codes.astype(np.uint8))
    big = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e30, -470.0, -1e9])
    np.testing.assert_array_equal(o.float_to_e4m3(big), [0x7E] * 6 + [0xFE] * 2)


def pin_e4m3_encode_nearest_even_brute_force(o):
    codes, vals = _finite_table()
    pos = vals[(vals > 0) & (codes < 0x80)]
    pos_codes = codes[(vals > 0) & (codes < 0x80)]
    order = np.argsort(pos)
    pos, pos_codes = pos[order], pos_codes[order]
    mids = (pos[:-1] + pos[1:]) / 2.0                       # exact ties
    rng = np.random.default_rng(61)
    rand = np.concatenate([rng.uniform(0, 448, 3000),
                           np.exp(rng.uniform(math.log(2.0 ** -12), math.log(440.0), 3000))])
    xs = np.concatenate([mids, rand, [0.0, 2.0 ** -10, 3 * 2.0 ** -11]]).astype(np.float32).astype(np.float64)
    got = o.float_to_e4m3(xs)
    allv = np.concatenate([[0.0], pos])
    allc = np.concatenate([[0], pos_codes])
    for x, g in zip(xs, got):
        d = np.abs(allv - x)
        best = np.flatnonzero(d == d.min())
        want = allc[best[0]] if len(best) == 1 else [c for c in allc[best] if c % 2 == 0][0]
        assert int(g) == int(want), (x, int(g), int(want))
    np.testing.assert_array_equal(o.float_to_e4m3(-xs), got | 0x80)
    # torch's float32 -> float8_e4m3fn is also round-to-nearest-even in range
    np.testing.assert_array_equal(got, _torch_encode(xs.astype(np.float32)))


# ---------------------------------------------------------- per-row scaling

def pin_quantize_row_invariants(o):
    rng = np.random.default_rng(62)
    for dtype in ("f16", "bf16"):
        x = normal_bits(rng, (40, 3, 64), dtype)
        codes, scales = o.quantize_e4m3_rows(x, dtype)
        assert codes.shape == x.shape and scales.shape == x.shape[:-1] and scales.dtype == np.float32
        xf = pa.bits_to_float64(x, dtype)
        amax = np.abs(xf).max(axis=-1)
        np.testing.assert_array_equal(scales, (amax.astype(np.float32) / np.float32(448)))
        # the largest element of each row is coded as +-448
        at = np.abs(xf).argmax(axis=-1)
        top = np.take_along_axis(codes, at[..., None], -1)[..., 0] & 0x7F
        assert (top == 0x7E).all()
        # round-to-nearest bound: half a step of the code grid, relative 2^-4
        # among normals, 2^-10 absolute among subnormals (plus float32 slack)
        y = xf / scales[..., None]
        err = np.abs(o.dequantize_e4m3_rows(codes, scales) - xf) / scales[..., None]
        bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 2.0 ** -20) + np.abs(y) * 2.0 ** -23
        assert (err <= bound).all()
        # sign symmetry
        neg = x ^ np.uint16(0x8000)
        c2, s2 = o.quantize_e4m3_rows(neg, dtype)
        np.testing.assert_array_equal(s2, scales)
        np.testing.assert_array_equal(c2, codes ^ 0x80)


def pin_quantize_power_of_two_scaling_and_zero_rows(o):
    rng = np.random.default_rng(63)
    x = normal_bits(rng, (16, 2, 32), "bf16")
    c1, s1 = o.quantize_e4m3_rows(x, "bf16")
    # times 2^5: bf16 exponent + 5 (no overflow for N(0,1) draws)
    x5 = (x.astype(np.uint32) + np.where((x & 0x7FFF) != 0, 5 << 7, 0)).astype(np.uint16)
    c5, s5 = o.quantize_e4m3_rows(x5, "bf16")
    np.testing.assert_array_equal(c5, c1)
    np.testing.assert_array_equal(s5, s1 * np.float32(32))
    z = np.zeros((2, 1, 8), np.uint16)
    z[1, 0, 3] = 0x8000                                  # a -0 survives as the -0 code
    cz, sz = o.quantize_e4m3_rows(z, "f16")
    np.testing.assert_array_equal(sz, np.ones((2, 1), np.float32))
    assert (cz[0] == 0).all() and cz[1, 0, 3] == 0x80 and (np.delete(cz[1, 0], 3) == 0).all()
    try:
        o.quantize_e4m3_rows(np.full((1, 1, 4), 0x7E00, np.uint16), "f16")
    except ValueError:
        pass
    else:
        raise AssertionError("a NaN row was quantised")


def tie_rows_f16():
    """fp16 rows whose float32 quotients x / s land exactly on E4M3 ties.

    Each row holds its amax ``A`` and ``+-x`` with ``x = 3 A 2^e``,
    e = -12..-2.  For these ``A`` the float32 scale ``fl32(A / 448)`` is a
    little below ``A / 448``, so the exact quotient ``x / s`` lies just above
    the midpoint ``21 * 2^(e+6)`` between two codes while its float32 rounding
    is the midpoint itself: only a float32 quotient followed by ties-to-even
    reproduces these codes.
    """
    rows = []
    for a_bits in (0x3802, 0x3806, 0x380A, 0x3810, 0x381E, 0x3834):
        a = float(np.uint16(a_bits).view(np.float16))
        xs = [3 * a * 2.0 ** e for e in range(-12, -1)]
        row = [a] + xs + [-x for x in xs[:4]]
        rows.append(np.array(row, np.float16).view(np.uint16))
    return np.stack(rows)[:, None, :]                  # [rows, 1 head, 16]


def pin_quantize_float32_quotient_ties(o):
    x = tie_rows_f16()
    codes, _ = o.quantize_e4m3_rows(x, "f16")
    xf = pa.bits_to_float64(x, "f16").astype(np.float32)
    s = (np.abs(xf).max(axis=-1) / np.float32(448)).astype(np.float32)
    q32 = (xf / s[..., None]).astype(np.float32)
    np.testing.assert_array_equal(codes, _torch_encode(q32))
    q64 = xf.astype(np.float64) / s[..., None].astype(np.float64)
    assert int((q64[..., 1:] > q32[..., 1:]).sum()) >= 60     # exact quotients sit past the ties


# ---------------------------------------- lossless inputs: the 16-bit oracle

def _lossless_bits(rng, shape, dtype):
    """Rows of E4M3 values times a per-row power of two, with one element of
    magnitude 448 * 2^k per row, so per-row quantisation is exact."""
    codes, vals = _finite_table()
    fin = vals[np.abs(vals) <= 448]
    x = rng.choice(fin, size=shape)
    k = rng.integers(-12, -5, size=shape[:-1])
    at = rng.integers(0, shape[-1], size=shape[:-1])
    np.put_along_axis(x, at[..., None], (448.0 * rng.choice([-1.0, 1.0], size=shape[:-1]))[..., None], -1)
    x = x * np.ldexp(1.0, k)[..., None]
    if dtype == "f16":
        bits = x.astype(np.float16).view(np.uint16)
    else:
        bits = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(pa.bits_to_float64(bits, dtype), x)  # exact in the 16-bit type
    return bits


def _fp8_pools(nb, hkv, d):
    kc = np.full((nb, 16, hkv, d), 0x7F, np.uint8)           # NaN codes
    ks = np.full((nb, hkv, 16), np.nan, np.float32)
    return kc, kc.copy(), ks, ks.copy()


def _live_slots(c):
    slots = []
    for b in range(c.block_tables.shape[0]):
        n = int(c.seq_lens[b]) if hasattr(c, "seq_lens") else int(c.ctx_lens[b] + c.q_lens[b])
        for p in range(n):
            slots.append(int(c.block_tables[b, p // 16]) * 16 + p % 16)
    return np.array(sorted(set(slots)), np.int64)


def pin_fp8_decode_lossless_equals_16bit(o):
    for dtype, hq, hkv in (("f16", 4, 2), ("bf16", 8, 2)):
        c = make_decode_case(name="pin", seed=64, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                             head_dim=16, seq_lens=[1, 15, 16, 17, 40, 0, 33], num_blocks=24,
                             max_blocks_per_seq=4, scale=0.25, write_last=False)
        rng = np.random.default_rng(65)
        slots = _live_slots(c)
        key = _lossless_bits(rng, (len(slots), hkv, 16), dtype)
        val = _lossless_bits(rng, (len(slots), hkv, 16), dtype)
        kc16, vc16 = pa.ref_reshape_and_cache(key, val, c.k_cache, c.v_cache, slots)
        want = pa.ref_decode(c.q, kc16, vc16, c.block_tables, c.seq_lens, c.scale, dtype)
        kc, vc, ks, vs = o.ref_reshape_and_cache_fp8(key, val, *_fp8_pools(24, hkv, 16), slots, dtype)
        got = o.ref_decode_fp8(c.q, kc, vc, ks, vs, c.block_tables, c.seq_lens, c.scale, dtype)
        np.testing.assert_array_equal(got, want)


def pin_fp8_prefill_lossless_equals_16bit(o):
    c = make_prefill_case(name="pin", seed=66, dtype="bf16", num_q_heads=6, num_kv_heads=2,
                          head_dim=16, q_lens=[5, 0, 17, 1, 33], ctx_lens=[0, 9, 20, 15, 40],
                          scale=0.25, extra_blocks=3)
    rng = np.random.default_rng(67)
    slots = _live_slots(c)
    key = _lossless_bits(rng, (len(slots), 2, 16), "bf16")
    val = _lossless_bits(rng, (len(slots), 2, 16), "bf16")
    kc16, vc16 = pa.ref_reshape_and_cache(key, val, c.k_cache, c.v_cache, slots)
    want = pa.ref_prefill_paged(c.q, kc16, vc16, c.block_tables, c.ctx_lens, c.query_start_loc,
                                c.scale, "bf16")
    kc, vc, ks, vs = o.ref_reshape_and_cache_fp8(key, val, *_fp8_pools(c.num_blocks, 2, 16), slots, "bf16")
    got = o.ref_prefill_paged_fp8(c.q, kc, vc, ks, vs, c.block_tables, c.ctx_lens,
                                  c.query_start_loc, c.scale, "bf16")
    np.testing.assert_array_equal(got, want)


def pin_fp8_reshape_semantics(o):
    rng = np.random.default_rng(68)
    key = normal_bits(rng, (3, 2, 8), "f16")
    val = normal_bits(rng, (3, 2, 8), "f16")
    slots = np.array([37, -1, 5], np.int64)
    pools = _fp8_pools(4, 2, 8)
    kc, vc, ks, vs = o.ref_reshape_and_cache_fp8(key, val, *pools, slots, "f16")
    kq, kscale = o.quantize_e4m3_rows(key, "f16")
    vq, vscale = o.quantize_e4m3_rows(val, "f16")
    np.testing.assert_array_equal(kc[2, 5], kq[0])
    np.testing.assert_array_equal(vc[0, 5], vq[2])
    np.testing.assert_array_equal(ks[2, :, 5], kscale[0])
    np.testing.assert_array_equal(vs[0, :, 5], vscale[2])
    assert {tuple(x) for x in np.argwhere((kc != pools[0]).any(axis=(2, 3)))} <= {(2, 5), (0, 5)}
    assert int(np.isfinite(ks).sum()) == 4 and int(np.isfinite(vs).sum()) == 4
    for bad in ([64, 0, 1], [5, 5, -1]):
        try:
            o.ref_reshape_and_cache_fp8(key, val, *pools, np.array(bad, np.int64), "f16")
        except (IndexError, ValueError):
            pass
        else:
            raise AssertionError(f"slots {bad} accepted")


def pin_fp8_scales_follow_the_block_table(o):
    """Moving blocks (codes and scales together) and rewriting the tables
    leaves the result unchanged; the scales are read per token and head."""
    c = make_decode_case(name="pin", seed=69, dtype="f16", num_q_heads=4, num_kv_heads=2,
                         head_dim=8, seq_lens=[30, 3, 47], num_blocks=10, max_blocks_per_seq=3,
                         scale=0.5, write_last=False)
    slots = _live_slots(c)
    rng = np.random.default_rng(70)
    key = normal_bits(rng, (len(slots), 2, 8), "f16")
    val = normal_bits(rng, (len(slots), 2, 8), "f16")
    kc, vc, ks, vs = o.ref_reshape_and_cache_fp8(key, val, *_fp8_pools(10, 2, 8), slots, "f16")
    base = o.ref_decode_fp8(c.q, kc, vc, ks, vs, c.block_tables, c.seq_lens, c.scale, "f16")
    assert np.isfinite(base).all()
    perm = rng.permutation(10)
    moved = [np.empty_like(a) for a in (kc, vc, ks, vs)]
    for m, a in zip(moved, (kc, vc, ks, vs)):
        m[perm] = a
    tables = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    np.testing.assert_array_equal(o.ref_decode_fp8(c.q, *moved, tables, c.seq_lens, c.scale, "f16"), base)
    # brute force for one sequence: dequantise token by token
    b, n = 2, 47
    k = np.stack([o.dequantize_e4m3_rows(kc[c.block_tables[b, p // 16], p % 16],
                                          ks[c.block_tables[b, p // 16], :, p % 16]) for p in range(n)])
    v = np.stack([o.dequantize_e4m3_rows(vc[c.block_tables[b, p // 16], p % 16],
                                          vs[c.block_tables[b, p // 16], :, p % 16]) for p in range(n)])
    want = pa.ref_contiguous_attention(pa.bits_to_float64(c.q[b], "f16")[None], k, v, c.scale,
                                       np.array([n - 1]))[0]
    np.testing.assert_allclose(base[b], want, rtol=0, atol=1e-13)


FP8_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
