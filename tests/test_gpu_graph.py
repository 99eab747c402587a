"""HIP-graph capture and replay of decode and prefill steps: cache write +
paged decode in 16-bit and FP8 caches, multi-query (verification) decode,
chunked prefill, and a decode step captured at a batch bucket and replayed
with fewer live sequences.

Graph mode keeps every tensor at a fixed address and changes only contents
between replays, the block table included; batches are padded up to a fixed
bucket size ("vLLM-Ascend 原理", §四, graph mode).  The library never
allocates, reads device memory on the host or memsets, so a captured step is
replayable as is.  Every replay is checked twice: against the float64 oracle
on host copies of the contents it ran on (q, k/v, tables, lengths, slots),
at the attention tolerance and bit-exactly for the cache pools; and against
the same step run eagerly, bit for bit.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (DecodeOnGPU, assert_close, dev_bits, dev_int, host_bits, host_f64,
                         require_gpu)
from workloads import make_decode_case, normal_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import paged_kv_cache_24_amd  # noqa: F401


def _capture(step):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    return graph


def _replay_then_eager(graph, step, out_graph, fresh):
    """Replay, then run the step eagerly into a fresh buffer; both host copies."""
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    eager = fresh()
    step(eager)
    torch.cuda.synchronize()
    return host_bits(out_graph).copy(), host_bits(eager)


@pytest.mark.parametrize("part", [64, -1])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("hq,hkv,dtype", [(8, 8, "f16"), (16, 2, "bf16")])
def test_captured_decode_step(hq, hkv, dtype, bs, part):
    """Cache write + split decode captured once; replayed with new q, shortened
    lengths (rollback) and two sequences trading table rows.  Fixed 64-token
    partitions (several per sequence: the merge runs too) or the balanced split
    (-1), whose stretch boundaries the kernels find from the lengths on the
    device at every replay."""
    import paged_kv_cache_24_amd as pa
    lens = [300, 17, 1, 129, 64, 0]
    c = make_decode_case(name="graph", seed=21, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                         head_dim=128, seq_lens=lens, num_blocks=64, max_blocks_per_seq=320 // bs,
                         scale=1 / math.sqrt(128), write_last=True, block_size=bs)
    g = DecodeOnGPU(c)
    kc, vc = oracle.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    need = pa.pa_decode_workspace_size(c.num_seqs, hq, hkv, 128, bs, c.max_blocks_per_seq, part)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out_graph = torch.empty_like(g.q)
    torch.cuda.synchronize()

    def step(out=out_graph):
        pa.pa_reshape_and_cache(g.key, g.value, g.k_cache, g.v_cache, g.slots)
        pa.pa_decode(out, g.q, g.k_cache, g.v_cache, g.tables, g.lens, c.scale, part, workspace=ws)

    graph = _capture(step)

    rng = np.random.default_rng(22)
    for replay in range(4):
        # new contents at the same addresses: q, lengths (a shorter sequence = rollback),
        # and block tables (two sequences trade rows)
        q = normal_bits(rng, tuple(g.q.shape), dtype)
        g.q.copy_(dev_bits(q, dtype))
        new_lens = np.array(lens, np.int32)
        new_lens[0] = 300 - 7 * replay
        tables = c.block_tables.copy()
        if replay % 2:
            tables[[1, 3]] = tables[[3, 1]]
            new_lens[[1, 3]] = new_lens[[3, 1]]
        g.lens.copy_(dev_int(new_lens))
        g.tables.copy_(dev_int(tables))
        got, eager = _replay_then_eager(graph, step, out_graph, lambda: torch.empty_like(g.q))
        np.testing.assert_array_equal(got, eager, err_msg=f"replay {replay}")
        np.testing.assert_array_equal(host_bits(g.k_cache), kc, err_msg=f"replay {replay}: K pool")
        np.testing.assert_array_equal(host_bits(g.v_cache), vc, err_msg=f"replay {replay}: V pool")
        ref = oracle.ref_decode(q, kc, vc, tables, new_lens, c.scale, dtype)
        assert_close(host_f64(out_graph), ref, dtype, f"replay {replay}")
        assert not (got[new_lens == 0] & 0x7FFF).any(), "an empty sequence must give zeros"


def test_captured_decode_step_fused_write():
    """pa_decode_step (the cache write inside the decode kernels) captured once and
    replayed with new key/value/q and lengths that advance by one token per
    replay, as a serving loop does: pools bit-exact vs the oracle's writes,
    outputs within tolerance, replay == eager."""
    import paged_kv_cache_24_amd as pa
    lens0 = np.array([40, 1, 16, 129, 63], np.int32)
    c = make_decode_case(name="graph-step", seed=25, dtype="f16", num_q_heads=8, num_kv_heads=8, head_dim=128,
                         seq_lens=lens0 + 4, num_blocks=48, max_blocks_per_seq=10, scale=1 / math.sqrt(128),
                         write_last=False)
    g = DecodeOnGPU(c)
    kc, vc = c.k_cache.copy(), c.v_cache.copy()
    key = torch.empty((c.num_seqs, 8, 128), dtype=torch.float16, device="cuda")
    value = torch.empty_like(key)
    g.lens.copy_(dev_int(lens0))
    out_graph = torch.empty_like(g.q)

    def step(out=out_graph):
        pa.pa_decode_step(out, g.q, key, value, g.k_cache, g.v_cache, g.tables, g.lens, c.scale, 0)

    rng = np.random.default_rng(26)
    graph = None
    for replay in range(4):
        lens = lens0 + replay
        kn = normal_bits(rng, (c.num_seqs, 8, 128), "f16")
        vn = normal_bits(rng, (c.num_seqs, 8, 128), "f16")
        q = normal_bits(rng, tuple(g.q.shape), "f16")
        key.copy_(dev_bits(kn, "f16"))
        value.copy_(dev_bits(vn, "f16"))
        g.q.copy_(dev_bits(q, "f16"))
        g.lens.copy_(dev_int(lens))
        # the oracle: each sequence's newest token written at position lens - 1, then the decode
        slots = np.array([int(c.block_tables[b, (n - 1) // 16]) * 16 + (n - 1) % 16 for b, n in enumerate(lens)],
                         np.int64)
        kc, vc = oracle.ref_reshape_and_cache(kn, vn, kc, vc, slots)
        ref = oracle.ref_decode(q, kc, vc, c.block_tables, lens, c.scale, "f16")
        if graph is None:
            pools = (g.k_cache.clone(), g.v_cache.clone())
            graph = _capture(step)                  # the warm-up and the capture ran the step once
            g.k_cache.copy_(pools[0])
            g.v_cache.copy_(pools[1])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(g.k_cache), kc, err_msg=f"replay {replay}: K pool")
        np.testing.assert_array_equal(host_bits(g.v_cache), vc, err_msg=f"replay {replay}: V pool")
        assert_close(host_f64(out_graph), ref, "f16", f"replay {replay}")
        eager = torch.empty_like(g.q)
        step(eager)                                 # rewrites the same rows with the same values
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(out_graph), host_bits(eager), err_msg=f"replay {replay}")


@pytest.mark.parametrize("fp8", [False, True])
def test_captured_shared_prefix_step(fp8):
    """pa_decode (pa_decode_fp8) with PA_DECODE_SHARED_PREFIX captured once: the
    sequence groups' shared runs are found on the device at every replay, so
    replays that change lengths, break a sharing run (one sequence's prefix
    copied to blocks of its own) and restore it all match the oracle."""
    # 8 q / 2 kv heads: waves of 4 sequences, aligned with the runs of 4 sharers
    import paged_kv_cache_24_amd as pa
    from gpu_helpers import Fp8DecodeOnGPU
    lens = [300, 17, 1, 129, 64, 0, 250, 200, 96, 33, 5]
    c = make_decode_case(name="graph-shared", seed=23, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                         head_dim=128, seq_lens=lens, num_blocks=96, max_blocks_per_seq=20,
                         scale=1 / math.sqrt(128), write_last=False, share_group=4, share_tokens=64)
    g = Fp8DecodeOnGPU(c) if fp8 else DecodeOnGPU(c)
    names = ("k_cache", "v_cache", "k_scales", "v_scales") if fp8 else ("k_cache", "v_cache")
    if fp8:
        g.write()
        host = dict(zip(names, (np.array(x) for x in g.oracle_pools())))   # the oracle's own FP8 write
        np.testing.assert_array_equal(g.k_cache.cpu().numpy(), host["k_cache"])
    else:
        host = {"k_cache": c.k_cache.copy(), "v_cache": c.v_cache.copy()}
    flags = pa.PA_DECODE_SHARED_PREFIX
    need = pa.pa_decode_workspace_size(c.num_seqs, 8, 2, 128, 16, c.max_blocks_per_seq, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out_graph = torch.empty_like(g.q)
    # four free blocks for the prefix copy of sequence 3
    used = set(c.block_tables[c.block_tables >= 0].tolist())
    free = [b for b in range(c.num_blocks) if b not in used][:4]
    assert len(free) == 4

    def step(out=out_graph):
        if fp8:
            pa.pa_decode_fp8(out, g.q, g.k_cache, g.v_cache, g.k_scales, g.v_scales, g.tables, g.lens,
                             c.scale, 0, workspace=ws, flags=flags)
        else:
            pa.pa_decode(out, g.q, g.k_cache, g.v_cache, g.tables, g.lens, c.scale, 0, workspace=ws,
                         flags=flags)

    graph = _capture(step)
    rng = np.random.default_rng(24)
    for replay in range(4):
        q = normal_bits(rng, tuple(g.q.shape), "bf16")
        g.q.copy_(dev_bits(q, "bf16"))
        new_lens = np.array(lens, np.int32)
        new_lens[0] = 300 - 9 * replay
        tables = c.block_tables.copy()
        if replay % 2:   # sequence 3 leaves its run: the prefix blocks copied to blocks of its own
            src = [int(b) for b in c.block_tables[3, :4]]
            for name in names:
                t = getattr(g, name)
                t[free] = t[src]
                host[name][free] = host[name][src]
            tables[3, :4] = free
        g.lens.copy_(dev_int(new_lens))
        g.tables.copy_(dev_int(tables))
        got, eager = _replay_then_eager(graph, step, out_graph, lambda: torch.empty_like(g.q))
        np.testing.assert_array_equal(got, eager, err_msg=f"replay {replay}")
        if fp8:
            ref = oracle.ref_decode_fp8(q, host["k_cache"], host["v_cache"], host["k_scales"], host["v_scales"],
                                        tables, new_lens, c.scale, "bf16")
        else:
            ref = oracle.ref_decode(q, host["k_cache"], host["v_cache"], tables, new_lens, c.scale, "bf16")
        assert_close(host_f64(out_graph), ref, "bf16", f"replay {replay}")


@pytest.mark.parametrize("fp8", [False, True])
def test_bucket_padded_decode_step(fp8):
    """A decode step captured once at a bucket of 8 sequences, then replayed
    with 5, 8, 3 and 1 live sequences: the rows past the live ones are padding
    with seq_len 0, slot -1 and table entries -1 (and NaN k/v, q), as graph mode
    pads a batch up to its bucket.  Each replay writes the last token of each
    live sequence; the pools must equal the oracle's cache write bit for bit
    (padding writes nothing), padded output rows must be exact zeros, and live
    rows must match the oracle's decode over the pools as they stand."""
    import paged_kv_cache_24_amd as pa
    bucket, dtype, hq, hkv, d = 8, "bf16", 16, 2, 128
    full_lens = np.array([300, 17, 1, 129, 64, 33, 250, 16], np.int32)
    c = make_decode_case(name="bucket", seed=41, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                         head_dim=d, seq_lens=full_lens, num_blocks=72, max_blocks_per_seq=20,
                         scale=1 / math.sqrt(d), write_last=True)
    assert len(c.slot_mapping) == bucket        # every sequence owns a last-token slot
    nan = np.uint16(0x7FC0)
    part = 64
    need = pa.pa_decode_workspace_size(bucket, hq, hkv, d, 16, c.max_blocks_per_seq, part)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    # fixed-address step inputs, sized for the bucket
    q_d = dev_bits(c.q, dtype)
    key_d = dev_bits(c.key, dtype)
    value_d = dev_bits(c.value, dtype)
    slots_d = dev_int(c.slot_mapping, torch.int64)
    tables_d = dev_int(c.block_tables)
    lens_d = dev_int(full_lens)
    out_graph = torch.empty_like(q_d)

    if fp8:
        # FP8 pools of every live token; the last tokens are written by the step
        kc16, vc16 = oracle.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache,
                                                  c.slot_mapping)
        pre = np.setdiff1d(_live_slots(c.block_tables, full_lens), c.slot_mapping)
        codes0 = np.full((c.num_blocks, 16, hkv, d), 0x7F, np.uint8)
        scales0 = np.full((c.num_blocks, hkv, 16), np.nan, np.float32)
        pools = list(oracle.ref_reshape_and_cache_fp8(
            kc16[pre // 16, pre % 16], vc16[pre // 16, pre % 16], codes0, codes0, scales0, scales0,
            pre, dtype))
        kd, vd, ksd, vsd = (torch.from_numpy(x).cuda() for x in pools)
    else:
        pools = [c.k_cache.copy(), c.v_cache.copy()]
        kd, vd = dev_bits(pools[0], dtype), dev_bits(pools[1], dtype)

    def step(out=out_graph):
        if fp8:
            pa.pa_reshape_and_cache_fp8(key_d, value_d, kd, vd, ksd, vsd, slots_d)
            pa.pa_decode_fp8(out, q_d, kd, vd, ksd, vsd, tables_d, lens_d, c.scale, part,
                             workspace=ws)
        else:
            pa.pa_reshape_and_cache(key_d, value_d, kd, vd, slots_d)
            pa.pa_decode(out, q_d, kd, vd, tables_d, lens_d, c.scale, part, workspace=ws)

    # capture on an all-padding batch (nothing is written or read while capturing)
    lens_d.zero_()
    slots_d.fill_(-1)
    tables_d.fill_(-1)
    graph = _capture(step)

    rng = np.random.default_rng(42)
    for replay, live in enumerate([5, 8, 3, 1]):
        pad = np.arange(bucket) >= live
        q = normal_bits(rng, tuple(q_d.shape), dtype)
        q[pad] = nan
        key = c.key.copy()
        value = c.value.copy()
        key[pad] = nan
        value[pad] = nan
        slots = np.where(pad, -1, c.slot_mapping).astype(np.int64)
        tables = np.where(pad[:, None], -1, c.block_tables).astype(np.int32)
        lens = np.where(pad, 0, full_lens).astype(np.int32)
        for dst, src in ((q_d, dev_bits(q, dtype)), (key_d, dev_bits(key, dtype)),
                         (value_d, dev_bits(value, dtype)), (slots_d, dev_int(slots, torch.int64)),
                         (tables_d, dev_int(tables)), (lens_d, dev_int(lens))):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = host_bits(out_graph).copy()
        what = f"{'fp8' if fp8 else 'bf16'} replay {replay} ({live} live of {bucket})"
        if fp8:
            # the oracle's quantiser refuses NaN rows: hand it the live rows only
            live_rows = ~pad
            pools = list(oracle.ref_reshape_and_cache_fp8(key[live_rows], value[live_rows], *pools,
                                                          slots[live_rows], dtype))
            for name, dev, want in zip(("K codes", "V codes", "K scales", "V scales"),
                                       (kd, vd, ksd, vsd), pools):
                np.testing.assert_array_equal(dev.cpu().numpy(), want, err_msg=f"{what}: {name}")
            ref = oracle.ref_decode_fp8(q, *pools, tables, lens, c.scale, dtype)
        else:
            pools = list(oracle.ref_reshape_and_cache(key, value, *pools, slots))
            np.testing.assert_array_equal(host_bits(kd), pools[0], err_msg=f"{what}: K pool")
            np.testing.assert_array_equal(host_bits(vd), pools[1], err_msg=f"{what}: V pool")
            ref = oracle.ref_decode(q, *pools, tables, lens, c.scale, dtype)
        assert not (got[pad] & 0x7FFF).any(), f"{what}: padded rows must be zeros"
        assert_close(host_f64(out_graph)[~pad], ref[~pad], dtype, what)
        eager = torch.empty_like(q_d)
        step(eager)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got, host_bits(eager), err_msg=f"{what}: eager")


def _live_slots(block_tables, lens):
    out = [block_tables[b, np.arange(int(n)) // 16].astype(np.int64) * 16 + np.arange(int(n)) % 16
           for b, n in enumerate(lens)]
    return np.unique(np.concatenate(out))


def test_captured_fp8_step():
    """FP8 cache write + FP8 decode (GQA, split) captured once, replayed with new
    q and new k contents."""
    import paged_kv_cache_24_amd as pa
    from gpu_helpers import Fp8DecodeOnGPU
    c = make_decode_case(name="graph-fp8", seed=23, dtype="bf16", num_q_heads=16, num_kv_heads=2,
                         head_dim=128, seq_lens=[300, 17, 1, 129, 64], num_blocks=64,
                         max_blocks_per_seq=20, scale=0.088, write_last=False)
    g = Fp8DecodeOnGPU(c)
    part = 64
    need = pa.pa_decode_workspace_size(c.num_seqs, 16, 2, 128, 16, c.max_blocks_per_seq, part)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out_graph = torch.empty_like(g.q)

    def step(out=out_graph):
        pa.pa_reshape_and_cache_fp8(g.key, g.value, g.k_cache, g.v_cache, g.k_scales, g.v_scales, g.slots)
        pa.pa_decode_fp8(out, g.q, g.k_cache, g.v_cache, g.k_scales, g.v_scales, g.tables, g.lens,
                         c.scale, part, workspace=ws)

    graph = _capture(step)
    rng = np.random.default_rng(24)
    for replay in range(3):
        q = normal_bits(rng, tuple(g.q.shape), "bf16")
        key = normal_bits(rng, tuple(g.key.shape), "bf16")
        g.q.copy_(dev_bits(q, "bf16"))
        g.key.copy_(dev_bits(key, "bf16"))
        got, eager = _replay_then_eager(graph, step, out_graph, lambda: torch.empty_like(g.q))
        np.testing.assert_array_equal(got, eager, err_msg=f"replay {replay}")
        pools = oracle.ref_reshape_and_cache_fp8(key, g.value_np, g.codes0, g.codes0, g.scales0,
                                                 g.scales0, g.slots_np, "bf16")
        for name, dev, want in zip(("K codes", "V codes", "K scales", "V scales"),
                                   (g.k_cache, g.v_cache, g.k_scales, g.v_scales), pools):
            np.testing.assert_array_equal(dev.cpu().numpy(), want, err_msg=f"replay {replay}: {name}")
        ref = oracle.ref_decode_fp8(q, *pools, c.block_tables, c.seq_lens, c.scale, "bf16")
        assert_close(host_f64(out_graph), ref, "bf16", f"fp8 replay {replay}")


def test_captured_verification_step():
    """Multi-query decode (4 draft queries per sequence) captured once and replayed
    with the sequence lengths shortened in place, as after rejected drafts."""
    import paged_kv_cache_24_amd as pa
    nq = 4
    lens = [300, 17, 2, 129]
    c = make_decode_case(name="graph-multi", seed=25, dtype="f16", num_q_heads=32, num_kv_heads=32,
                         head_dim=128, seq_lens=lens, num_blocks=64, max_blocks_per_seq=20,
                         scale=0.088, write_last=False)
    g = DecodeOnGPU(c)
    rng = np.random.default_rng(26)
    qm = dev_bits(normal_bits(rng, (c.num_seqs, nq, 32, 128), "f16"), "f16")
    part = 64
    need = pa.pa_decode_workspace_size(c.num_seqs * nq, 32, 32, 128, 16, c.max_blocks_per_seq, part)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out_graph = torch.empty_like(qm)

    def step(out=out_graph):
        pa.pa_decode_multi(out, qm, g.k_cache, g.v_cache, g.tables, g.lens, c.scale, part, workspace=ws)

    graph = _capture(step)
    for replay in range(3):
        new_lens = np.maximum(np.array(lens) - 3 * replay, 0).astype(np.int32)
        q = normal_bits(rng, tuple(qm.shape), "f16")
        g.lens.copy_(dev_int(new_lens))
        qm.copy_(dev_bits(q, "f16"))
        got, eager = _replay_then_eager(graph, step, out_graph, lambda: torch.empty_like(qm))
        np.testing.assert_array_equal(got, eager, err_msg=f"replay {replay}")
        ref = oracle.ref_decode_multi(q, c.k_cache, c.v_cache, c.block_tables, new_lens, c.scale, "f16")
        assert_close(host_f64(out_graph), ref, "f16", f"verification replay {replay}")


def test_captured_verification_step_balanced():
    """The same capture in the balanced split: the default partition takes it for a
    multi-query call where its partial states fit the workspace documented for the
    call, as here (128 sequences with 2048-token tables, 8 q heads per kv head, so
    32 (query, head) columns per kv head in two chunks; the sizes of the
    two-chunk case of tests/test_gpu_multi.py)."""
    import paged_kv_cache_24_amd as pa
    nq, hq, hkv = 4, 16, 2
    rng = np.random.default_rng(28)
    lens = rng.integers(0, 301, 128)
    lens[:4] = [0, 1, 16, 300]
    c = make_decode_case(name="graph-multi-balanced", seed=29, dtype="f16", num_q_heads=hq,
                         num_kv_heads=hkv, head_dim=128, seq_lens=lens,
                         num_blocks=int(sum((n + 15) // 16 for n in lens)) + 4, max_blocks_per_seq=128,
                         scale=1 / math.sqrt(128), write_last=False)
    g = DecodeOnGPU(c)
    qm = dev_bits(normal_bits(rng, (c.num_seqs, nq, hq, 128), "f16"), "f16")
    part = 0
    need = pa.pa_decode_workspace_size(c.num_seqs * nq, hq, hkv, 128, 16, c.max_blocks_per_seq, part)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out_graph = torch.empty_like(qm)

    def step(out=out_graph):
        pa.pa_decode_multi(out, qm, g.k_cache, g.v_cache, g.tables, g.lens, c.scale, part, workspace=ws)

    graph = _capture(step)
    for replay in range(3):
        new_lens = np.maximum(lens - 5 * replay, 0).astype(np.int32)
        q = normal_bits(rng, tuple(qm.shape), "f16")
        g.lens.copy_(dev_int(new_lens))
        qm.copy_(dev_bits(q, "f16"))
        got, eager = _replay_then_eager(graph, step, out_graph, lambda: torch.empty_like(qm))
        np.testing.assert_array_equal(got, eager, err_msg=f"replay {replay}")
        ref = oracle.ref_decode_multi(q, c.k_cache, c.v_cache, c.block_tables, new_lens, c.scale, "f16")
        assert_close(host_f64(out_graph), ref, "f16", f"balanced verification replay {replay}")


def test_captured_prefill_step():
    """Cache write + chunked prefill captured once, replayed with new q and new
    k/v and with the cached-context lengths shortened in place."""
    import paged_kv_cache_24_amd as pa
    from gpu_helpers import PrefillOnGPU
    from workloads import make_prefill_case
    ctx = [40, 0, 300]
    c = make_prefill_case(name="graph-prefill", seed=27, dtype="bf16", num_q_heads=8,
                          num_kv_heads=2, head_dim=128, q_lens=[70, 1, 33], ctx_lens=ctx,
                          scale=0.088)
    g = PrefillOnGPU(c)
    out_graph = torch.zeros_like(g.q)

    def step(out=out_graph):
        pa.pa_reshape_and_cache(g.key, g.value, g.k_cache, g.v_cache, g.slots)
        pa.pa_prefill_paged(out, g.q, g.k_cache, g.v_cache, g.tables, g.ctx, g.qsl, c.scale,
                            c.max_q_len)

    graph = _capture(step)
    rng = np.random.default_rng(28)
    for replay in range(3):
        q = normal_bits(rng, tuple(g.q.shape), "bf16")
        key = normal_bits(rng, tuple(g.key.shape), "bf16")
        value = normal_bits(rng, tuple(g.value.shape), "bf16")
        # a shorter cached context: the rows see fewer keys (the slots written stay valid)
        new_ctx = np.maximum(np.array(ctx) - 16 * replay, 0).astype(np.int32)
        g.q.copy_(dev_bits(q, "bf16"))
        g.key.copy_(dev_bits(key, "bf16"))
        g.value.copy_(dev_bits(value, "bf16"))
        g.ctx.copy_(dev_int(new_ctx))
        got, eager = _replay_then_eager(graph, step, out_graph, lambda: torch.zeros_like(g.q))
        np.testing.assert_array_equal(got, eager, err_msg=f"replay {replay}")
        kc, vc = oracle.ref_reshape_and_cache(key, value, c.k_cache, c.v_cache, c.slot_mapping)
        np.testing.assert_array_equal(host_bits(g.k_cache), kc, err_msg=f"replay {replay}: K pool")
        ref = oracle.ref_prefill_paged(q, kc, vc, c.block_tables, new_ctx, c.query_start_loc,
                                       c.scale, "bf16")
        assert_close(host_f64(out_graph), ref, "bf16", f"prefill replay {replay}")
