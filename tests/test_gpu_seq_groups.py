"""Sequence groups of the matrix-core decode (PA_DECODE_SHARED_PREFIX).

With the flag, pa_decode lets one wave carry the q heads of S = 16 / group
consecutive sequences through the leading blocks they share (read once for
all of them); the balanced split runs over those shared runs and every
sequence's own blocks.  Checked against the float64 oracle: groups of 3 to 8 q heads
per kv head (S = 5 to 2), sharing patterns cut across the waves on purpose
(prefix runs of 3 or 16 sequences against waves of 2 to 5 sequences), a
ragged last group, empty sequences, sequences shorter than the prefix, and
hand-built tables for the edges of the shared run: every sequence sharing all
of its blocks, sharing that ends where fewer than two sequences remain,
sharing broken and resumed, shared runs of 1 to 3 blocks.  The same over the
FP8 cache (pa_decode_fp8) against the oracle's FP8 decode.  Where no block is
shared the flagged call takes exactly the unflagged balanced split's path and
must match it bit for bit; everywhere the result must not depend on where the
pool's blocks sit."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (DecodeOnGPU, Fp8DecodeOnGPU, TOL, assert_close, dev_bits, dev_int, host_bits, host_f64,
                         require_gpu)
from workloads import DecodeCase, decode_gqa_shared_prefix, make_decode_case, normal_bits

pytestmark = pytest.mark.gpu

LENS = [0, 1, 15, 16, 17, 40, 100, 255, 256, 257, 300, 511, 700, 0, 33, 64, 129]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import paged_kv_cache_24_amd  # noqa: F401


def _flag():
    import paged_kv_cache_24_amd as pa
    return pa.PA_DECODE_SHARED_PREFIX


def _case(dtype, group, hkv, share_group, share_tokens=256, lens=LENS, seed=0):
    need = sum((n + 15) // 16 for n in lens) + 4
    return make_decode_case(name=f"seqgrp-{dtype}-g{group}-h{hkv}-s{share_group}", seed=900 + seed + group,
                            dtype=dtype, num_q_heads=group * hkv, num_kv_heads=hkv, head_dim=128,
                            seq_lens=lens, num_blocks=need, max_blocks_per_seq=48,
                            scale=1 / math.sqrt(128), write_last=False, share_group=share_group,
                            share_tokens=share_tokens if share_group else 0)


def _ref(c):
    return oracle.ref_decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, c.scale, c.dtype)


def _check(c, parts=(0, -1)):
    g = DecodeOnGPU(c)
    ref = _ref(c)
    for part in parts:
        out = host_f64(g.decode(partition_tokens=part, flags=_flag()))
        assert_close(out, ref, c.dtype, f"{c.name} partition={part}")
    return g


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("group,hkv", [(3, 2), (4, 2), (5, 1), (8, 2), (4, 8)])
@pytest.mark.parametrize("share_group", [0, 3, 16])
def test_groups_match_oracle(dtype, group, hkv, share_group):
    _check(_case(dtype, group, hkv, share_group))


@pytest.mark.parametrize("group", [6, 7])
def test_groups_of_two_sequences(group):
    """Groups 6 and 7 leave 4 and 2 of the 16 columns unused."""
    _check(_case("bf16", group, 2, 4, share_tokens=128, seed=group))


@pytest.mark.parametrize("group,hkv", [(3, 2), (4, 2), (8, 1)])
def test_no_shared_block_equals_balanced_bit_exact(group, hkv):
    """No block shared: the groups take nothing and the balanced split all, as unflagged."""
    c = _case("bf16", group, hkv, 0)
    g = DecodeOnGPU(c)
    a = host_bits(g.decode(partition_tokens=-1)).copy()
    np.testing.assert_array_equal(a, host_bits(g.decode(flags=_flag())))


def _explicit_case(name, tables, lens, group=4, hkv=2, dtype="bf16", seed=0):
    """A pool of finite values everywhere and block tables given by hand."""
    rng = np.random.default_rng(seed)
    tables = np.asarray(tables, np.int32)
    nb = int(tables.max()) + 1
    d = 128
    return DecodeCase(name=name, dtype=dtype, num_q_heads=group * hkv, num_kv_heads=hkv, head_dim=d,
                      num_blocks=nb, max_blocks_per_seq=tables.shape[1], scale=1 / math.sqrt(d),
                      q=normal_bits(rng, (len(lens), group * hkv, d), dtype),
                      k_cache=normal_bits(rng, (nb, 16, hkv, d), dtype),
                      v_cache=normal_bits(rng, (nb, 16, hkv, d), dtype),
                      block_tables=tables, seq_lens=np.asarray(lens, np.int32),
                      key=np.zeros((0, hkv, d), np.uint16), value=np.zeros((0, hkv, d), np.uint16),
                      slot_mapping=np.zeros(0, np.int64))


def _rows(*rows, width=12):
    out = np.full((len(rows), width), -1, np.int32)
    for i, r in enumerate(rows):
        out[i, :len(r)] = r
    return out


SHARE = list(range(10))


@pytest.mark.parametrize("name,tables,lens", [
    # one group of 4: every sequence shares every block, equal lengths
    ("all-shared", _rows(SHARE, SHARE, SHARE, SHARE), [160, 160, 160, 160]),
    # the same table, different lengths: sharing ends where one sequence remains
    ("lengths", _rows(SHARE, SHARE, SHARE, SHARE), [5, 40, 100, 160]),
    # broken at block 4, equal again at 5..: the run stops at 4
    ("broken", _rows(SHARE, SHARE[:4] + [20] + SHARE[5:], SHARE, SHARE), [160, 150, 140, 130]),
    # runs of 1, 2 and 3 blocks: ranges left empty
    ("run1", _rows([0, 11], [0, 12], [0, 13], [0, 14]), [30, 32, 20, 17]),
    ("run2", _rows([0, 1, 11], [0, 1, 12], [0, 1, 13], [0, 1, 14]), [40, 48, 33, 45]),
    ("run3", _rows([0, 1, 2, 11], [0, 1, 2, 12], [0, 1, 2, 13], [0, 1, 2, 14]), [60, 64, 49, 50]),
    # two groups, an empty sequence in play nowhere, a 1-token sequence
    ("two-groups", _rows(SHARE, SHARE, [], SHARE, [15, 16, 17], [15, 16, 18], [15], [15, 16, 19]),
     [150, 160, 0, 1, 40, 48, 3, 37]),
    # only the first two of the group share: blocks stay private (the run needs all in play)
    ("partial", _rows(SHARE, SHARE, [20, 21, 22], [23, 24, 25]), [160, 160, 40, 41]),
])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_shared_run_edges(name, tables, lens, dtype):
    c = _explicit_case(f"edge-{name}-{dtype}", tables, lens, dtype=dtype, seed=len(name))
    _check(c)


@pytest.mark.parametrize("group", [3, 5, 8])
def test_shared_run_edges_other_groups(group):
    """Waves of 5, 3 and 2 sequences over one table shared by 6 sequences."""
    tables = _rows(*([SHARE] * 6), [30, 31], [32])
    c = _explicit_case(f"edge-g{group}", tables, [160, 17, 90, 160, 33, 1, 20, 9], group=group, hkv=1,
                       seed=group)
    _check(c)


def test_both_flags_together():
    """The streaming hint only changes how K/V is loaded, not a bit of the result."""
    import paged_kv_cache_24_amd as pa
    c = _case("bf16", 4, 2, 16)
    g = DecodeOnGPU(c)
    a = host_bits(g.decode(flags=pa.PA_DECODE_SHARED_PREFIX)).copy()
    b = host_bits(g.decode(flags=pa.PA_DECODE_SHARED_PREFIX | pa.PA_DECODE_STREAM_KV))
    np.testing.assert_array_equal(a, b)


def test_flag_has_no_effect_elsewhere():
    """Fixed partitions, head_dim 64, 2 or 16 q heads per kv head, pa_decode_partitions:
    the flag is accepted and changes nothing."""
    import paged_kv_cache_24_amd as pa
    for group, hkv, d, part in ((4, 2, 128, 64), (4, 2, 64, 0), (2, 4, 128, 0), (16, 1, 128, 0)):
        c = make_decode_case(name="noeffect", seed=950 + group + d, dtype="bf16",
                             num_q_heads=group * hkv, num_kv_heads=hkv, head_dim=d,
                             seq_lens=LENS, num_blocks=sum((n + 15) // 16 for n in LENS) + 4,
                             max_blocks_per_seq=48, scale=0.1, write_last=False)
        g = DecodeOnGPU(c)
        a = host_bits(g.decode(partition_tokens=part)).copy()
        b = host_bits(g.decode(partition_tokens=part, flags=pa.PA_DECODE_SHARED_PREFIX))
        np.testing.assert_array_equal(a, b, err_msg=f"group {group} hkv {hkv} d {d} part {part}")
    c = _case("bf16", 4, 2, 16)
    g = DecodeOnGPU(c)
    need = pa.pa_decode_workspace_size(c.num_seqs, c.num_q_heads, c.num_kv_heads, 128, 16, 48, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    outs = []
    for flags in (0, pa.PA_DECODE_SHARED_PREFIX):
        out = torch.empty_like(g.q)
        pa.pa_decode_partitions(out, g.q, g.k_cache, g.v_cache, g.tables, g.lens, c.scale, ws, flags=flags)
        pa.pa_decode_merge(out, g.lens, c.num_kv_heads, 48, ws)
        outs.append(host_bits(out).copy())
    np.testing.assert_array_equal(outs[0], outs[1])


def test_shared_prefix_close_to_private_copies():
    """The same contexts with every block copied out: no sharing, the unflagged
    balanced path; the two agree to the decode tolerance."""
    c = decode_gqa_shared_prefix(batch=20, max_len=1024, min_len=16, group=8, prefix=512)
    g = DecodeOnGPU(c)
    shared = host_f64(g.decode(flags=_flag())).copy()
    nb = int((c.block_tables >= 0).sum())
    kc = np.empty((nb,) + c.k_cache.shape[1:], np.uint16)
    vc = np.empty_like(kc)
    tables = np.full_like(c.block_tables, -1)
    cur = 0
    for b in range(c.num_seqs):
        for j, blk in enumerate(c.block_tables[b]):
            if blk < 0:
                break
            kc[cur], vc[cur] = c.k_cache[blk], c.v_cache[blk]
            tables[b, j] = cur
            cur += 1
    g.k_cache, g.v_cache, g.tables = dev_bits(kc, c.dtype), dev_bits(vc, c.dtype), dev_int(tables)
    private = host_bits(g.decode(flags=_flag())).copy()
    np.testing.assert_array_equal(private, host_bits(g.decode(partition_tokens=-1)))
    assert np.abs(shared - host_f64(g.decode(partition_tokens=-1))).max() <= TOL[c.dtype]


def test_block_permutation_invariance_bit_exact():
    c = decode_gqa_shared_prefix(batch=19, max_len=1024, min_len=16, group=4, prefix=256)
    g = DecodeOnGPU(c)
    base = host_bits(g.decode(flags=_flag())).copy()
    perm = np.random.default_rng(81).permutation(c.num_blocks)
    kc = np.empty_like(c.k_cache)
    vc = np.empty_like(c.v_cache)
    kc[perm] = c.k_cache
    vc[perm] = c.v_cache
    tables = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    g.k_cache, g.v_cache, g.tables = dev_bits(kc, c.dtype), dev_bits(vc, c.dtype), dev_int(tables)
    moved = host_bits(g.decode(flags=_flag()))
    np.testing.assert_array_equal(base, moved)


def test_deterministic_repeat():
    c = decode_gqa_shared_prefix(batch=24, max_len=2048, min_len=16, group=4, prefix=512)
    g = DecodeOnGPU(c)
    a = host_bits(g.decode(flags=_flag())).copy()
    for _ in range(3):
        np.testing.assert_array_equal(a, host_bits(g.decode(flags=_flag())))


def test_noalloc_with_flag_equals_pa_decode():
    import paged_kv_cache_24_amd as pa
    c = _case("bf16", 4, 2, 16)
    g = DecodeOnGPU(c)
    a = host_bits(g.decode(flags=pa.PA_DECODE_SHARED_PREFIX)).copy()
    out = torch.empty_like(g.q)
    pa.pa_decode_noalloc(out, g.q, g.k_cache, g.v_cache, g.tables, g.lens, c.scale,
                         flags=pa.PA_DECODE_SHARED_PREFIX)
    np.testing.assert_array_equal(a, host_bits(out))


def _check_fp8(c, parts=(0, -1)):
    import oracle
    g = Fp8DecodeOnGPU(c)
    g.write()
    kc, vc, ks, vs = g.oracle_pools()
    ref = oracle.ref_decode_fp8(c.q, kc, vc, ks, vs, c.block_tables, c.seq_lens, c.scale, c.dtype)
    for part in parts:
        out = host_f64(g.decode(partition_tokens=part, flags=_flag()))
        assert_close(out, ref, c.dtype, f"fp8 {c.name} partition={part}")
    return g


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("group,hkv", [(3, 2), (4, 2), (8, 1)])
@pytest.mark.parametrize("share_group", [0, 3, 16])
def test_fp8_groups_match_oracle(dtype, group, hkv, share_group):
    _check_fp8(_case(dtype, group, hkv, share_group))


@pytest.mark.parametrize("name,tables,lens", [
    ("all-shared", _rows(SHARE, SHARE, SHARE, SHARE), [160, 160, 160, 160]),
    ("lengths", _rows(SHARE, SHARE, SHARE, SHARE), [5, 40, 100, 160]),
    ("broken", _rows(SHARE, SHARE[:4] + [20] + SHARE[5:], SHARE, SHARE), [160, 150, 140, 130]),
    ("run1", _rows([0, 11], [0, 12], [0, 13], [0, 14]), [30, 32, 20, 17]),
    ("run3", _rows([0, 1, 2, 11], [0, 1, 2, 12], [0, 1, 2, 13], [0, 1, 2, 14]), [60, 64, 49, 50]),
    ("two-groups", _rows(SHARE, SHARE, [], SHARE, [15, 16, 17], [15, 16, 18], [15], [15, 16, 19]),
     [150, 160, 0, 1, 40, 48, 3, 37]),
])
def test_fp8_shared_run_edges(name, tables, lens):
    _check_fp8(_explicit_case(f"fp8-edge-{name}", tables, lens, seed=len(name) + 7))


def test_fp8_no_shared_block_equals_balanced_bit_exact():
    c = _case("bf16", 4, 2, 0)
    g = Fp8DecodeOnGPU(c)
    g.write()
    a = host_bits(g.decode(partition_tokens=-1)).copy()
    np.testing.assert_array_equal(a, host_bits(g.decode(flags=_flag())))


def test_fp8_block_permutation_invariance_bit_exact():
    c = decode_gqa_shared_prefix(batch=19, max_len=1024, min_len=16, group=4, prefix=256)
    g = Fp8DecodeOnGPU(c)
    g.write()
    base = host_bits(g.decode(flags=_flag())).copy()
    perm = np.random.default_rng(82).permutation(c.num_blocks)
    inv = torch.from_numpy(np.argsort(perm)).cuda()
    # move every pool block b to perm[b]
    for name in ("k_cache", "v_cache", "k_scales", "v_scales"):
        t = getattr(g, name)
        setattr(g, name, t[inv].contiguous())
    tables = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    g.tables = dev_int(tables)
    moved = host_bits(g.decode(flags=_flag()))
    np.testing.assert_array_equal(base, moved)
