"""HIP-graph capture and replay of decode steps: cache write + paged decode in
16-bit and FP8 caches, and multi-query (verification) decode.

Graph mode keeps every tensor at a fixed address and changes only contents
between replays, the block table included ("vLLM-Ascend 原理", §四, graph mode).
The library never allocates, reads device memory on the host or memsets, so a
captured step must equal the eager step on every replay, with the contents of
q, the tables and the lengths rewritten in place between replays.
"""

import math

import numpy as np
import pytest
import torch

from gpu_helpers import DecodeOnGPU, dev_bits, dev_int, host_bits, require_gpu
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


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("hq,hkv,dtype", [(8, 8, "f16"), (16, 2, "bf16")])
def test_captured_decode_step_matches_eager(hq, hkv, dtype, bs):
    import paged_kv_cache_24_amd as pa
    lens = [300, 17, 1, 129, 64, 0]
    c = make_decode_case(name="graph", seed=21, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                         head_dim=128, seq_lens=lens, num_blocks=64, max_blocks_per_seq=320 // bs,
                         scale=1 / math.sqrt(128), write_last=True, block_size=bs)
    g = DecodeOnGPU(c)
    part = 64                                   # several partitions: exercises the merge too
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
        g.q.copy_(dev_bits(normal_bits(rng, tuple(g.q.shape), dtype), dtype))
        new_lens = np.array(lens, np.int32)
        new_lens[0] = 300 - 7 * replay
        g.lens.copy_(dev_int(new_lens))
        tables = c.block_tables.copy()
        if replay % 2:
            tables[[1, 3]] = tables[[3, 1]]
            new_lens[[1, 3]] = new_lens[[3, 1]]
            g.lens.copy_(dev_int(new_lens))
        g.tables.copy_(dev_int(tables))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = torch.empty_like(g.q)
        step(eager)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(out_graph), host_bits(eager),
                                      err_msg=f"replay {replay}")


def test_captured_fp8_step_matches_eager():
    """FP8 cache write + FP8 decode (GQA, split) captured once, replayed with new
    q and new k/v contents; every replay equals the eager step bit for bit."""
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
        g.q.copy_(dev_bits(normal_bits(rng, tuple(g.q.shape), "bf16"), "bf16"))
        g.key.copy_(dev_bits(normal_bits(rng, tuple(g.key.shape), "bf16"), "bf16"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = torch.empty_like(g.q)
        step(eager)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(out_graph), host_bits(eager), err_msg=f"replay {replay}")


def test_captured_verification_step_matches_eager():
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
        g.lens.copy_(dev_int(np.maximum(np.array(lens) - 3 * replay, 0).astype(np.int32)))
        qm.copy_(dev_bits(normal_bits(rng, tuple(qm.shape), "f16"), "f16"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = torch.empty_like(qm)
        step(eager)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(out_graph), host_bits(eager), err_msg=f"replay {replay}")


def test_captured_prefill_step_matches_eager():
    """Cache write + chunked prefill captured once, replayed with new q and new
    k/v and with the cached-context lengths shortened in place; every replay
    equals the eager step bit for bit."""
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
        g.q.copy_(dev_bits(normal_bits(rng, tuple(g.q.shape), "bf16"), "bf16"))
        g.key.copy_(dev_bits(normal_bits(rng, tuple(g.key.shape), "bf16"), "bf16"))
        g.value.copy_(dev_bits(normal_bits(rng, tuple(g.value.shape), "bf16"), "bf16"))
        # a shorter cached context: the rows see fewer keys (the slots written stay valid)
        g.ctx.copy_(dev_int(np.maximum(np.array(ctx) - 16 * replay, 0).astype(np.int32)))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = torch.zeros_like(g.q)
        step(eager)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(out_graph), host_bits(eager), err_msg=f"replay {replay}")
