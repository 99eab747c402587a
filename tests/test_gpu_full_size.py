"""Parity at the workloads' full sizes, in the launch configuration the bench
times (default partition length), checked on sampled outputs the oracle
computes one sequence at a time."""

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
