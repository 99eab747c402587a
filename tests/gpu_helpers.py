"""Shared helpers of the GPU tests: move workloads to the device and back,
compare with the oracle.  Tolerances: max-abs error 2e-3 for fp16 outputs and
1e-2 for bf16 outputs against the float64 oracle."""

from __future__ import annotations

import numpy as np
import torch

TOL = {"f16": 2e-3, "bf16": 1e-2}
TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16}


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev_bits(arr: np.ndarray, dtype: str) -> torch.Tensor:
    """uint16 bit patterns -> device tensor of the 16-bit float type."""
    t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
    return t.to("cuda").view(TORCH_DTYPE[dtype])


def dev_int(arr: np.ndarray, dtype=torch.int32) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dtype).to("cuda")


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().double().numpy()


class DecodeOnGPU:
    """A decode workload resident on the GPU."""

    def __init__(self, case):
        self.case = case
        dt = case.dtype
        self.q = dev_bits(case.q, dt)
        self.k_cache = dev_bits(case.k_cache, dt)
        self.v_cache = dev_bits(case.v_cache, dt)
        self.key = dev_bits(case.key, dt)
        self.value = dev_bits(case.value, dt)
        self.slots = dev_int(case.slot_mapping, torch.int64)
        self.tables = dev_int(case.block_tables)
        self.lens = dev_int(case.seq_lens)
        self.out = torch.empty_like(self.q)

    def write(self):
        import paged_kv_cache_24_amd as pa
        pa.pa_reshape_and_cache(self.key, self.value, self.k_cache, self.v_cache, self.slots)

    def decode(self, partition_tokens=0, out=None, flags=0):
        import paged_kv_cache_24_amd as pa
        out = self.out if out is None else out
        pa.pa_decode(out, self.q, self.k_cache, self.v_cache, self.tables, self.lens,
                     self.case.scale, partition_tokens, flags=flags)
        return out


class PrefillOnGPU:
    def __init__(self, case):
        self.case = case
        dt = case.dtype
        self.q = dev_bits(case.q, dt)
        self.k_cache = dev_bits(case.k_cache, dt)
        self.v_cache = dev_bits(case.v_cache, dt)
        self.key = dev_bits(case.key, dt)
        self.value = dev_bits(case.value, dt)
        self.slots = dev_int(case.slot_mapping, torch.int64)
        self.tables = dev_int(case.block_tables)
        self.ctx = dev_int(case.ctx_lens)
        self.qsl = dev_int(case.query_start_loc)
        self.out = torch.zeros_like(self.q)

    def write(self):
        import paged_kv_cache_24_amd as pa
        pa.pa_reshape_and_cache(self.key, self.value, self.k_cache, self.v_cache, self.slots)

    def prefill(self, out=None):
        import paged_kv_cache_24_amd as pa
        out = self.out if out is None else out
        pa.pa_prefill_paged(out, self.q, self.k_cache, self.v_cache, self.tables, self.ctx,
                            self.qsl, self.case.scale, max(self.case.max_q_len, 1))
        return out


def ulps(got64: np.ndarray, ref64: np.ndarray, dtype: str) -> np.ndarray:
    """|got - ref| in units of the spacing of the output type at |ref| (fp16:
    10 fraction bits, normals from 2^-14; bf16: 7 fraction bits)."""
    frac, emin = (10, -14) if dtype == "f16" else (7, -126)
    mag = np.maximum(np.abs(ref64), 2.0 ** emin)
    spacing = 2.0 ** (np.floor(np.log2(mag)) - frac)
    return np.abs(got64 - ref64) / spacing


def assert_close(got64: np.ndarray, ref64: np.ndarray, dtype: str, what: str = ""):
    assert got64.shape == ref64.shape, (got64.shape, ref64.shape)
    assert np.isfinite(got64).all(), f"{what}: non-finite output"
    err = np.abs(got64 - ref64)
    worst = float(err.max()) if err.size else 0.0
    if worst > TOL[dtype]:
        i = np.unravel_index(int(np.argmax(err)), err.shape)
        u = ulps(got64, ref64, dtype)
        raise AssertionError(
            f"{what}: max-abs error {worst:.3e} > {TOL[dtype]} at {tuple(int(x) for x in i)} "
            f"(ref {ref64[i]:.4f}, {u[i]:.2f} ulps of {dtype} there; max |ref| "
            f"{np.abs(ref64).max():.3f}, max error {u.max():.2f} ulps)")
    return worst


# unit roundoff of the probabilities the matrix-core paths feed to PV (rounded to
# the output's 16-bit type before the product); the vector paths keep them in float32
U_MFMA = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
EPS32 = 2.0 ** -13


def weighted_sums(q64, k64, v64, pos, scale, ref):
    """sum_j w_j |v_j - ref| and sum_j w_j |v_j| for every row, head and element,
    w the softmax weights of the row's visible keys (the oracle's attention
    applied to |V - ref| and |V|).  q64 [L, Hq, D], k64/v64 [n, Hkv, D] float64,
    pos [L] the rows' positions, ref [L, Hq, D] the oracle's outputs."""
    import oracle
    lq, hq, _ = q64.shape
    group = hq // k64.shape[1]
    mag = oracle.ref_contiguous_attention(q64, k64, np.abs(v64), scale, pos)
    dev = np.empty_like(ref)
    for i in range(lq):
        for h in range(hq):
            g = h // group
            dev[i, h] = oracle.ref_contiguous_attention(
                q64[i:i + 1, h:h + 1], k64[:, g:g + 1], np.abs(v64[:, g:g + 1] - ref[i, h]), scale,
                pos[i:i + 1])[0, 0]
    return dev, mag


def rounding_bound(ref, dtype, dev, mag, u):
    """What the arithmetic of a path guarantees: half a spacing of the output type
    (the final rounding), the weights' rounding to 16 bits (relative u each; the
    row sums add the rounded weights, so they still sum to one) acting on the
    spread of V around the output, and float32 accumulation."""
    frac, emin = (10, -14) if dtype == "f16" else (7, -126)
    spacing = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** emin))) - frac)
    return 0.5 * spacing + 2 * u / (1 - 2 * u) * dev + EPS32 * mag


def assert_close_or_bound(got64, ref64, dtype, bound_fn, what=""):
    """The stated tolerance, except where the rounding of the path's arithmetic
    alone can exceed it (short contexts with outputs of magnitude ~2 and more on
    the matrix-core paths): there the element must meet ``bound_fn()``, computed
    only when needed.  Returns the number of elements held to the bound."""
    assert got64.shape == ref64.shape, (got64.shape, ref64.shape)
    assert np.isfinite(got64).all(), f"{what}: non-finite output"
    err = np.abs(got64 - ref64)
    over = err > TOL[dtype]
    if not over.any():
        return 0
    bound = bound_fn()
    bad = over & (err > bound)
    if bad.any():
        i = np.unravel_index(int(np.argmax(np.where(bad, err / bound, 0))), err.shape)
        raise AssertionError(
            f"{what}: error {err[i]:.3e} above the tolerance {TOL[dtype]} and above the rounding "
            f"bound {bound[i]:.3e} at {tuple(int(x) for x in i)} (ref {ref64[i]:.4f}, "
            f"{ulps(got64, ref64, dtype)[i]:.2f} ulps)")
    print(f"{what}: {int(over.sum())} element(s) above {TOL[dtype]} (worst {err.max():.3e}, "
          f"{ulps(got64, ref64, dtype)[over].max():.2f} ulps), all within the rounding bound", flush=True)
    return int(over.sum())


def live_slots(block_tables: np.ndarray, lens: np.ndarray) -> np.ndarray:
    """Sorted distinct slots of every token the sequences hold (shared
    blocks counted once)."""
    out = []
    for b in range(block_tables.shape[0]):
        p = np.arange(int(lens[b]))
        out.append(block_tables[b, p // 16].astype(np.int64) * 16 + p % 16)
    return np.unique(np.concatenate(out)) if out else np.zeros(0, np.int64)


class Fp8DecodeOnGPU:
    """A decode workload over an FP8 cache: the 16-bit pools of a DecodeCase
    (after its cache write) give the k/v of every live token, which the FP8
    cache write quantises into code pools that start as NaN codes (0x7F) with
    NaN scales, so nothing unwritten can go unnoticed."""

    def __init__(self, case, slots=None):
        import oracle
        self.case = case
        dt = case.dtype
        kc16, vc16 = oracle.ref_reshape_and_cache(case.key, case.value, case.k_cache, case.v_cache,
                                                  case.slot_mapping)
        self.slots_np = live_slots(case.block_tables, case.seq_lens) if slots is None else slots
        blk, off = self.slots_np // 16, self.slots_np % 16
        self.key_np = np.ascontiguousarray(kc16[blk, off])
        self.value_np = np.ascontiguousarray(vc16[blk, off])
        nb, hkv, d = case.num_blocks, case.num_kv_heads, case.head_dim
        self.codes0 = np.full((nb, 16, hkv, d), 0x7F, np.uint8)
        self.scales0 = np.full((nb, hkv, 16), np.nan, np.float32)
        self.q = dev_bits(case.q, dt)
        self.key = dev_bits(self.key_np, dt)
        self.value = dev_bits(self.value_np, dt)
        self.slots = dev_int(self.slots_np, torch.int64)
        self.k_cache = torch.from_numpy(self.codes0).cuda()
        self.v_cache = torch.from_numpy(self.codes0).cuda()
        self.k_scales = torch.from_numpy(self.scales0).cuda()
        self.v_scales = torch.from_numpy(self.scales0).cuda()
        self.tables = dev_int(case.block_tables)
        self.lens = dev_int(case.seq_lens)
        self.out = torch.empty_like(self.q)

    def write(self):
        import paged_kv_cache_24_amd as pa
        pa.pa_reshape_and_cache_fp8(self.key, self.value, self.k_cache, self.v_cache, self.k_scales,
                                    self.v_scales, self.slots)

    def oracle_pools(self):
        import oracle
        return oracle.ref_reshape_and_cache_fp8(self.key_np, self.value_np, self.codes0, self.codes0,
                                                self.scales0, self.scales0, self.slots_np,
                                                self.case.dtype)

    def decode(self, partition_tokens=0, out=None, flags=0):
        import paged_kv_cache_24_amd as pa
        out = self.out if out is None else out
        pa.pa_decode_fp8(out, self.q, self.k_cache, self.v_cache, self.k_scales, self.v_scales,
                         self.tables, self.lens, self.case.scale, partition_tokens, flags=flags)
        return out


class Fp8PrefillOnGPU:
    """A chunked-prefill workload over an FP8 cache: every token the chunk
    reads (cached context and the chunk's own) is quantised by the FP8 cache
    write from the case's 16-bit k/v, into NaN-poisoned code and scale pools."""

    def __init__(self, case):
        import oracle
        self.case = case
        dt = case.dtype
        kc16, vc16 = oracle.ref_reshape_and_cache(case.key, case.value, case.k_cache, case.v_cache,
                                                  case.slot_mapping)
        lens = case.ctx_lens.astype(np.int64) + case.q_lens.astype(np.int64)
        self.slots_np = live_slots(case.block_tables, lens)
        blk, off = self.slots_np // 16, self.slots_np % 16
        self.key_np = np.ascontiguousarray(kc16[blk, off])
        self.value_np = np.ascontiguousarray(vc16[blk, off])
        nb, hkv, d = case.num_blocks, case.num_kv_heads, case.head_dim
        self.codes0 = np.full((nb, 16, hkv, d), 0x7F, np.uint8)
        self.scales0 = np.full((nb, hkv, 16), np.nan, np.float32)
        self.q = dev_bits(case.q, dt)
        self.key = dev_bits(self.key_np, dt)
        self.value = dev_bits(self.value_np, dt)
        self.slots = dev_int(self.slots_np, torch.int64)
        self.k_cache = torch.from_numpy(self.codes0).cuda()
        self.v_cache = torch.from_numpy(self.codes0).cuda()
        self.k_scales = torch.from_numpy(self.scales0).cuda()
        self.v_scales = torch.from_numpy(self.scales0).cuda()
        self.tables = dev_int(case.block_tables)
        self.ctx = dev_int(case.ctx_lens)
        self.qsl = dev_int(case.query_start_loc)
        self.out = torch.zeros_like(self.q)

    def write(self):
        import paged_kv_cache_24_amd as pa
        pa.pa_reshape_and_cache_fp8(self.key, self.value, self.k_cache, self.v_cache, self.k_scales,
                                    self.v_scales, self.slots)

    def oracle_pools(self):
        import oracle
        return oracle.ref_reshape_and_cache_fp8(self.key_np, self.value_np, self.codes0, self.codes0,
                                                self.scales0, self.scales0, self.slots_np,
                                                self.case.dtype)

    def prefill(self, out=None):
        import paged_kv_cache_24_amd as pa
        out = self.out if out is None else out
        pa.pa_prefill_paged_fp8(out, self.q, self.k_cache, self.v_cache, self.k_scales, self.v_scales,
                                self.tables, self.ctx, self.qsl, self.case.scale,
                                max(self.case.max_q_len, 1))
        return out
