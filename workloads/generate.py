"""Seeded generators for the five paged-attention workloads.

Recipe (the same for every workload):

* Values are N(0, 1) float32 draws from ``numpy.random.default_rng`` rounded
  to the storage type with round-to-nearest-even (fp16 through numpy, bf16 by
  integer rounding of the float32 bits).  Arrays are returned as raw
  ``uint16`` bit patterns so every consumer sees identical bits.
* Each sequence draws its K and V from its own generator seeded with
  ``[seed, stream, sequence]``; sizes, permutations and q come from
  ``default_rng(seed)`` in a fixed order.  Results do not depend on how many
  threads fill the pool.
* Physical blocks are handed out from ``rng.permutation(num_blocks)`` in
  order, ``ceil(tokens / block_size)`` per sequence (the host allocator of
  the ``PagedKVCache`` sketch), and every block-table entry past a sequence's
  last block is -1.  Blocks hold 16 tokens unless ``block_size`` says
  otherwise (32 is the other usual size); the values drawn do not depend on
  it, so one seed gives the same tokens in either layout.
* Every slot that no sequence reads holds NaN, so a kernel that reads past a
  sequence's end cannot go unnoticed.
* A token whose k/v the cache-write step stores has NaN in the pool beforehand
  and its k/v in ``key``/``value``; its slot is
  ``physical_block * block_size + offset``, the slot convention of the
  cache-write call.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

NAN_BITS = {"f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}
BLOCK_SIZE = 16

# stream tags for per-sequence generators
_K, _V, _NEWK, _NEWV, _SHK, _SHV, _Q = 1, 2, 3, 4, 5, 6, 7


def _to_bits(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        b = x32.view(np.uint32)
        return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
                >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


def normal_bits(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) draws rounded to ``dtype``, as uint16 bit patterns."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    chunk = 1 << 22
    buf = np.empty(min(chunk, max(n, 1)), np.float32)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        rng.standard_normal(out=buf[:m], dtype=np.float32)
        out[s:s + m] = _to_bits(buf[:m], dtype)
    return out.reshape(shape)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _place(pool: np.ndarray, blocks: np.ndarray, data: np.ndarray, nan: np.uint16):
    """Copy ``data`` (``[n, Hkv, D]``) into whole physical ``blocks`` in order;
    the unused tail of the last block gets NaN."""
    n = data.shape[0]
    nb = len(blocks)
    bs = pool.shape[1]
    if nb == 0:
        return
    padded = np.full((nb * bs,) + data.shape[1:], nan, np.uint16)
    padded[:n] = data
    pool[blocks] = padded.reshape((nb, bs) + data.shape[1:])


def _ceil_blocks(n: int, block_size: int = BLOCK_SIZE) -> int:
    return (n + block_size - 1) // block_size


@dataclass
class DecodeCase:
    """Inputs of one decode step.  All arrays are host numpy arrays.

    The pool arrays hold the state *before* the cache write; ``key``/``value``
    with ``slot_mapping`` are the tokens the cache write stores (possibly none).
    ``seq_lens`` counts those tokens too.
    """
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    q: np.ndarray               # uint16 [B, Hq, D]
    k_cache: np.ndarray         # uint16 [NB, block_size, Hkv, D]
    v_cache: np.ndarray
    block_tables: np.ndarray    # int32 [B, MB], -1 padded
    seq_lens: np.ndarray        # int32 [B]
    key: np.ndarray             # uint16 [N, Hkv, D]
    value: np.ndarray
    slot_mapping: np.ndarray    # int64 [N]
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def block_size(self) -> int:
        return int(self.k_cache.shape[1])

    def kv_bytes(self) -> int:
        """K+V bytes of all live tokens (each kv head's tile counted once)."""
        return int(self.seq_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * self.head_dim * 2


@dataclass
class PrefillCase:
    """Inputs of one chunked-prefill step (cache write, then attention)."""
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    q: np.ndarray               # uint16 [T, Hq, D]
    k_cache: np.ndarray         # uint16 [NB, block_size, Hkv, D], before the cache write
    v_cache: np.ndarray
    block_tables: np.ndarray    # int32 [B, MB]
    ctx_lens: np.ndarray        # int32 [B]
    query_start_loc: np.ndarray  # int32 [B + 1]
    key: np.ndarray             # uint16 [T, Hkv, D]
    value: np.ndarray
    slot_mapping: np.ndarray    # int64 [T]
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc)

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def block_size(self) -> int:
        return int(self.k_cache.shape[1])


def make_decode_case(*, name: str, seed: int, dtype: str, num_q_heads: int,
                     num_kv_heads: int, head_dim: int, seq_lens, num_blocks: int,
                     max_blocks_per_seq: int, scale: float, write_last: bool,
                     share_group: int = 0, share_tokens: int = 0,
                     rng: np.random.Generator | None = None,
                     perm: np.ndarray | None = None, block_size: int = BLOCK_SIZE) -> DecodeCase:
    """Build a decode workload.

    ``share_group > 0`` makes each run of ``share_group`` consecutive sequences
    point at the same physical blocks for their first ``share_tokens`` tokens
    (a shared prefix); past it each sequence has private blocks.  With sharing
    the pool needs no cache write (a write into a shared block would need a
    copy first), so ``write_last`` must be False.
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, np.int64)
    b_count = len(seq_lens)
    hkv, d = num_kv_heads, head_dim
    nan = NAN_BITS[dtype]
    if share_group and write_last:
        raise ValueError("shared-prefix workloads carry no cache write")
    if share_group and share_tokens % block_size:
        raise ValueError("the shared prefix must be whole blocks")

    # allocation: hand out physical blocks in permutation order
    if perm is None:
        perm = rng.permutation(num_blocks)
    tables = np.full((b_count, max_blocks_per_seq), -1, np.int32)
    cursor = 0
    shared_blocks = {}
    for b in range(b_count):
        nb = _ceil_blocks(int(seq_lens[b]), block_size)
        if nb > max_blocks_per_seq:
            raise ValueError(f"sequence {b} needs {nb} blocks > {max_blocks_per_seq}")
        if share_group:
            grp = b // share_group
            n_shared = share_tokens // block_size
            if grp not in shared_blocks:
                shared_blocks[grp] = perm[cursor:cursor + n_shared]
                cursor += n_shared
            own = max(0, nb - n_shared)
            tables[b, :min(nb, n_shared)] = shared_blocks[grp][:min(nb, n_shared)]
            tables[b, n_shared:n_shared + own] = perm[cursor:cursor + own]
            cursor += own
        else:
            tables[b, :nb] = perm[cursor:cursor + nb]
            cursor += nb
        if cursor > num_blocks:
            raise ValueError("pool too small for the sequences")

    q = normal_bits(np.random.default_rng([seed, _Q]), (b_count, num_q_heads, d), dtype)
    k_cache = np.full((num_blocks, block_size, hkv, d), nan, np.uint16)
    v_cache = np.full_like(k_cache, nan)

    n_written = 1 if write_last else 0

    def fill_seq(b):
        n = int(seq_lens[b])
        start = share_tokens if share_group else 0
        n_own = max(0, n - n_written - start)
        if n_own == 0 and not (share_group and n > start):
            return
        kd = normal_bits(np.random.default_rng([seed, _K, b]), (n_own, hkv, d), dtype)
        vd = normal_bits(np.random.default_rng([seed, _V, b]), (n_own, hkv, d), dtype)
        nb_total = _ceil_blocks(n, block_size)
        first = start // block_size
        blocks = tables[b, first:nb_total]
        _place(k_cache, blocks, kd, nan)
        _place(v_cache, blocks, vd, nan)

    def fill_group(grp):
        members = range(grp * share_group, min(b_count, (grp + 1) * share_group))
        longest = max(int(seq_lens[b]) for b in members)
        n = min(share_tokens, longest)
        kd = normal_bits(np.random.default_rng([seed, _SHK, grp]), (n, hkv, d), dtype)
        vd = normal_bits(np.random.default_rng([seed, _SHV, grp]), (n, hkv, d), dtype)
        blocks = shared_blocks[grp][:_ceil_blocks(n, block_size)]
        _place(k_cache, blocks, kd, nan)
        _place(v_cache, blocks, vd, nan)

    with ThreadPoolExecutor(_threads()) as ex:
        if share_group:
            list(ex.map(fill_group, sorted(shared_blocks)))
        list(ex.map(fill_seq, range(b_count)))

    # tokens stored by the cache-write step: the last token of each non-empty sequence
    writers = [b for b in range(b_count) if write_last and seq_lens[b] > 0]
    key = np.empty((len(writers), hkv, d), np.uint16)
    value = np.empty_like(key)
    slots = np.empty(len(writers), np.int64)
    for i, b in enumerate(writers):
        pos = int(seq_lens[b]) - 1
        key[i] = normal_bits(np.random.default_rng([seed, _NEWK, b]), (hkv, d), dtype)
        value[i] = normal_bits(np.random.default_rng([seed, _NEWV, b]), (hkv, d), dtype)
        slots[i] = int(tables[b, pos // block_size]) * block_size + pos % block_size

    return DecodeCase(name=name, dtype=dtype, num_q_heads=num_q_heads,
                      num_kv_heads=hkv, head_dim=d, num_blocks=num_blocks,
                      max_blocks_per_seq=max_blocks_per_seq,
                      scale=float(np.float32(scale)), q=q, k_cache=k_cache,
                      v_cache=v_cache, block_tables=tables,
                      seq_lens=seq_lens.astype(np.int32), key=key, value=value,
                      slot_mapping=slots,
                      meta={"seed": seed, "blocks_used": cursor,
                            "share_group": share_group, "share_tokens": share_tokens})


def make_prefill_case(*, name: str, seed: int, dtype: str, num_q_heads: int,
                      num_kv_heads: int, head_dim: int, q_lens, ctx_lens, scale: float,
                      extra_blocks: int = 0, max_blocks_per_seq: int | None = None,
                      rng: np.random.Generator | None = None,
                      block_size: int = BLOCK_SIZE) -> PrefillCase:
    """Build a chunked-prefill workload: sequence ``b`` has ``ctx_lens[b]``
    tokens already cached and ``q_lens[b]`` new tokens, packed back to back."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, np.int64)
    ctx_lens = np.asarray(ctx_lens, np.int64)
    b_count = len(q_lens)
    hkv, d = num_kv_heads, head_dim
    nan = NAN_BITS[dtype]
    nbs = [_ceil_blocks(int(c + l), block_size) for c, l in zip(ctx_lens, q_lens)]
    num_blocks = sum(nbs) + extra_blocks
    mb = max_blocks_per_seq if max_blocks_per_seq is not None else max(max(nbs, default=1), 1)
    perm = rng.permutation(num_blocks)
    tables = np.full((b_count, mb), -1, np.int32)
    cursor = 0
    for b in range(b_count):
        tables[b, :nbs[b]] = perm[cursor:cursor + nbs[b]]
        cursor += nbs[b]
    qsl = np.zeros(b_count + 1, np.int64)
    qsl[1:] = np.cumsum(q_lens)
    t = int(qsl[-1])

    q = normal_bits(np.random.default_rng([seed, _Q]), (t, num_q_heads, d), dtype)
    k_cache = np.full((num_blocks, block_size, hkv, d), nan, np.uint16)
    v_cache = np.full_like(k_cache, nan)
    key = np.empty((t, hkv, d), np.uint16)
    value = np.empty_like(key)

    def fill_seq(b):
        c = int(ctx_lens[b])
        kd = normal_bits(np.random.default_rng([seed, _K, b]), (c, hkv, d), dtype)
        vd = normal_bits(np.random.default_rng([seed, _V, b]), (c, hkv, d), dtype)
        _place(k_cache, tables[b, :_ceil_blocks(c, block_size)], kd, nan)
        _place(v_cache, tables[b, :_ceil_blocks(c, block_size)], vd, nan)
        lo, hi = int(qsl[b]), int(qsl[b + 1])
        key[lo:hi] = normal_bits(np.random.default_rng([seed, _NEWK, b]), (hi - lo, hkv, d), dtype)
        value[lo:hi] = normal_bits(np.random.default_rng([seed, _NEWV, b]), (hi - lo, hkv, d), dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill_seq, range(b_count)))

    slots = np.empty(t, np.int64)
    for b in range(b_count):
        lo = int(qsl[b])
        pos = int(ctx_lens[b]) + np.arange(int(q_lens[b]))
        slots[lo:lo + len(pos)] = (tables[b, pos // block_size].astype(np.int64) * block_size +
                                   pos % block_size)

    return PrefillCase(name=name, dtype=dtype, num_q_heads=num_q_heads,
                       num_kv_heads=hkv, head_dim=d, num_blocks=num_blocks,
                       max_blocks_per_seq=mb, scale=float(np.float32(scale)),
                       q=q, k_cache=k_cache, v_cache=v_cache, block_tables=tables,
                       ctx_lens=ctx_lens.astype(np.int32),
                       query_start_loc=qsl.astype(np.int32), key=key, value=value,
                       slot_mapping=slots, meta={"seed": seed})


# --------------------------------------------------------------------------
# The five workloads.  ``batch`` and friends shrink a workload for tests while
# keeping its structure (head counts, dtype, length distribution, sharing).
# --------------------------------------------------------------------------

def decode_tiny(seed: int = 1) -> DecodeCase:
    """Batch 4, 4 q = 4 kv heads, head_dim 64, fp16, lengths 1/17/33/100, a
    64-block pool handed out by a seeded permutation, scale 1/8; the last token
    of each sequence goes through the cache write."""
    return make_decode_case(name="decode_tiny", seed=seed, dtype="f16", num_q_heads=4,
                            num_kv_heads=4, head_dim=64, seq_lens=[1, 17, 33, 100],
                            num_blocks=64, max_blocks_per_seq=7, scale=1 / 8,
                            write_last=True)


def decode_llama2_7b_layer(seed: int = 2, batch: int = 64, max_len: int = 4096,
                           num_heads: int = 32, write_last: bool = True,
                           block_size: int = BLOCK_SIZE) -> DecodeCase:
    """One LLaMA-2-7B-shaped attention layer at decode: 32 q = 32 kv heads,
    head_dim 128, fp16, lengths uniform in [512, max_len], a pool of
    batch x max_len / block_size blocks (2^31 bytes per K pool at full size)."""
    rng = np.random.default_rng(seed)
    lo = min(512, max_len)
    lens = rng.integers(lo, max_len + 1, batch)
    mb = max_len // block_size
    return make_decode_case(name="decode_llama2_7b_layer", seed=seed, dtype="f16",
                            num_q_heads=num_heads, num_kv_heads=num_heads, head_dim=128,
                            seq_lens=lens, num_blocks=batch * mb, max_blocks_per_seq=mb,
                            scale=1 / math.sqrt(128), write_last=write_last, rng=rng,
                            block_size=block_size)


def decode_gqa_shared_prefix(seed: int = 3, batch: int = 256, max_len: int = 8192,
                             min_len: int = 128, group: int = 16,
                             prefix: int = 1024, block_size: int = BLOCK_SIZE) -> DecodeCase:
    """GQA decode, 32 q / 8 kv heads, head_dim 128, bf16, lengths log-uniform
    in [min_len, max_len]; each run of ``group`` sequences shares the physical
    blocks of a ``prefix``-token prefix, then diverges into private blocks."""
    rng = np.random.default_rng(seed)
    lens = np.floor(np.exp(rng.uniform(math.log(min_len), math.log(max_len), batch))).astype(np.int64)
    lens = np.clip(lens, min_len, max_len)
    n_groups = (batch + group - 1) // group
    private = sum(max(0, _ceil_blocks(int(n), block_size) - prefix // block_size) for n in lens)
    nb = n_groups * (prefix // block_size) + private
    return make_decode_case(name="decode_gqa_shared_prefix", seed=seed, dtype="bf16",
                            num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=lens,
                            num_blocks=nb, max_blocks_per_seq=max_len // block_size,
                            scale=1 / math.sqrt(128), write_last=False,
                            share_group=group, share_tokens=prefix, rng=rng,
                            block_size=block_size)


def prefill_chunked(seed: int = 4, batch: int = 16, new_tokens: int = 8192,
                    max_ctx: int = 4096, block_size: int = BLOCK_SIZE) -> PrefillCase:
    """Chunked prefill: ``new_tokens`` new tokens split over ``batch``
    sequences by a multinomial draw, cached context uniform in [0, max_ctx],
    32 q / 8 kv heads, head_dim 128, bf16, causal."""
    rng = np.random.default_rng(seed)
    q_lens = rng.multinomial(new_tokens, [1.0 / batch] * batch)
    ctx = rng.integers(0, max_ctx + 1, batch)
    return make_prefill_case(name="prefill_chunked", seed=seed, dtype="bf16", num_q_heads=32,
                             num_kv_heads=8, head_dim=128, q_lens=q_lens, ctx_lens=ctx,
                             scale=1 / math.sqrt(128), rng=rng, block_size=block_size)


def decode_long_context(seed: int = 5, batch: int = 8, seq_len: int = 65536,
                        num_blocks: int = 40000) -> DecodeCase:
    """Long-context decode: 64 q / 8 kv heads, head_dim 128, bf16, every
    sequence ``seq_len`` tokens, blocks scattered over a ``num_blocks`` pool."""
    rng = np.random.default_rng(seed)
    mb = seq_len // BLOCK_SIZE
    perm = rng.permutation(num_blocks)
    return make_decode_case(name="decode_long_context", seed=seed, dtype="bf16",
                            num_q_heads=64, num_kv_heads=8, head_dim=128,
                            seq_lens=[seq_len] * batch, num_blocks=num_blocks,
                            max_blocks_per_seq=mb, scale=1 / math.sqrt(128),
                            write_last=False, rng=rng, perm=perm)


CONFIG_BUILDERS = {
    "decode_tiny": decode_tiny,
    "decode_llama2_7b_layer": decode_llama2_7b_layer,
    "decode_gqa_shared_prefix": decode_gqa_shared_prefix,
    "prefill_chunked": prefill_chunked,
    "decode_long_context": decode_long_context,
}
