"""HIP-graph capture and replay of a decode step (cache write + paged decode).

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


@pytest.mark.parametrize("hq,hkv,dtype", [(8, 8, "f16"), (16, 2, "bf16")])
def test_captured_decode_step_matches_eager(hq, hkv, dtype):
    import paged_kv_cache_24_amd as pa
    lens = [300, 17, 1, 129, 64, 0]
    c = make_decode_case(name="graph", seed=21, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                         head_dim=128, seq_lens=lens, num_blocks=64, max_blocks_per_seq=20,
                         scale=1 / math.sqrt(128), write_last=True)
    g = DecodeOnGPU(c)
    part = 64                                   # several partitions: exercises the merge too
    need = pa.pa_decode_workspace_size(c.num_seqs, hq, hkv, 128, c.max_blocks_per_seq, part)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out_graph = torch.empty_like(g.q)
    torch.cuda.synchronize()

    def step(out):
        pa.pa_reshape_and_cache(g.key, g.value, g.k_cache, g.v_cache, g.slots)
        pa.pa_decode(out, g.q, g.k_cache, g.v_cache, g.tables, g.lens, c.scale, part, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out_graph)                         # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(out_graph)

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
