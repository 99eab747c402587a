"""Invariants of the seeded workload generators (CPU only)."""

import numpy as np

from workloads import (NAN_BITS, decode_gqa_shared_prefix, decode_llama2_7b_layer, decode_tiny,
                       make_decode_case, prefill_chunked)


def _read_slots(tables, lens, bs=16):
    """(block, offset) pairs some sequence reads, by walking whole blocks."""
    read = set()
    for row, n in zip(tables, lens):
        for j in range((int(n) + bs - 1) // bs):
            for off in range(min(bs, int(n) - bs * j)):
                read.add((int(row[j]), off))
    return read


def _check_pool(case, lens, written):
    nan = NAN_BITS[case.dtype]
    bs = case.k_cache.shape[1]
    read = _read_slots(case.block_tables, lens, bs)
    nb = case.k_cache.shape[0]
    for blk in range(nb):
        for off in range(bs):
            is_nan = (case.k_cache[blk, off] == nan).all() and (case.v_cache[blk, off] == nan).all()
            if (blk, off) in read and (blk, off) not in written:
                assert not (case.k_cache[blk, off] == nan).any(), (blk, off)
            else:
                assert is_nan, (blk, off)


def test_decode_tiny_layout():
    c = decode_tiny()
    assert list(c.seq_lens) == [1, 17, 33, 100]
    assert c.k_cache.shape == (64, 16, 4, 64) and c.q.shape == (4, 4, 64)
    assert c.scale == 0.125 and c.dtype == "f16"
    used = c.block_tables[c.block_tables >= 0]
    assert len(used) == 1 + 2 + 3 + 7 and len(set(used.tolist())) == len(used)
    assert (c.block_tables[0, 1:] == -1).all()
    written = {(int(s) // 16, int(s) % 16) for s in c.slot_mapping}
    assert len(written) == 4
    _check_pool(c, c.seq_lens, written)
    # each written slot is the last token of its sequence
    for i, b in enumerate(range(4)):
        pos = int(c.seq_lens[b]) - 1
        assert c.slot_mapping[i] == c.block_tables[b, pos // 16] * 16 + pos % 16


def test_decode_seeded_and_deterministic():
    a = decode_llama2_7b_layer(batch=3, max_len=256, num_heads=2)
    b = decode_llama2_7b_layer(batch=3, max_len=256, num_heads=2)
    for x, y in [(a.q, b.q), (a.k_cache, b.k_cache), (a.block_tables, b.block_tables)]:
        np.testing.assert_array_equal(x, y)
    c = decode_llama2_7b_layer(seed=9, batch=3, max_len=256, num_heads=2)
    assert not np.array_equal(a.q, c.q)


def test_shared_prefix_layout():
    c = decode_gqa_shared_prefix(batch=32, max_len=2048, min_len=128, group=16, prefix=1024)
    for grp in range(2):
        rows = c.block_tables[grp * 16:(grp + 1) * 16]
        lens = c.seq_lens[grp * 16:(grp + 1) * 16]
        for r, n in zip(rows, lens):
            k = min(64, (int(n) + 15) // 16)
            np.testing.assert_array_equal(r[:k], rows[np.argmax(lens)][:k])
    _check_pool(c, c.seq_lens, set())
    assert c.num_blocks == int(len(np.unique(c.block_tables[c.block_tables >= 0])))


def test_prefill_layout():
    c = prefill_chunked(batch=4, new_tokens=100, max_ctx=40)
    assert c.q.shape[0] == 100 == int(c.query_start_loc[-1])
    assert (np.diff(c.query_start_loc) >= 0).all()
    written = {(int(s) // 16, int(s) % 16) for s in c.slot_mapping}
    assert len(written) == 100
    _check_pool(c, c.ctx_lens + c.q_lens, written)


def test_empty_and_block_multiple_lengths():
    c = make_decode_case(name="t", seed=5, dtype="bf16", num_q_heads=2, num_kv_heads=1,
                         head_dim=64, seq_lens=[0, 16, 32, 1], num_blocks=8,
                         max_blocks_per_seq=2, scale=0.125, write_last=True)
    assert (c.block_tables[0] == -1).all()
    assert len(c.slot_mapping) == 3
    _check_pool(c, c.seq_lens, {(int(s) // 16, int(s) % 16) for s in c.slot_mapping})


def test_block32_layout():
    """32-token blocks: the same tokens as the 16-token layout of one seed,
    read slot for slot through either table."""
    kw = dict(name="t", seed=6, dtype="f16", num_q_heads=2, num_kv_heads=2, head_dim=64,
              seq_lens=[0, 31, 32, 33, 70], scale=0.125, write_last=True)
    a = make_decode_case(num_blocks=12, max_blocks_per_seq=5, **kw)
    b = make_decode_case(num_blocks=7, max_blocks_per_seq=3, block_size=32, **kw)
    assert b.k_cache.shape == (7, 32, 2, 64) and b.block_size == 32 and a.block_size == 16
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.key, b.key)
    used = b.block_tables[b.block_tables >= 0]
    assert len(used) == 0 + 1 + 1 + 2 + 3 and len(set(used.tolist())) == len(used)
    for i, s in enumerate(b.slot_mapping):
        blk, off = int(s) // 32, int(s) % 32
        seq = [x for x in range(5) if b.seq_lens[x] > 0][i]
        pos = int(b.seq_lens[seq]) - 1
        assert (blk, off) == (int(b.block_tables[seq, pos // 32]), pos % 32)
    _check_pool(b, b.seq_lens, {(int(s) // 32, int(s) % 32) for s in b.slot_mapping})
    for seq in range(5):
        for pos in range(int(b.seq_lens[seq]) - 1):   # the cached tokens
            np.testing.assert_array_equal(
                a.k_cache[a.block_tables[seq, pos // 16], pos % 16],
                b.k_cache[b.block_tables[seq, pos // 32], pos % 32])
