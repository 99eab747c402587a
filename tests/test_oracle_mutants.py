"""Plant plausible mistakes in copies of the oracle and check the pins catch them.

Each mutant is the oracle's own source with one edit (a dropped term, a wrong
index, a swapped operand...), loaded as a separate module on the CPU.  A pin
set that lets a mutant through would not be pinning the oracle.
"""

import os
import types

import pytest

import oracle.paged_attention as oracle_mod
from oracle_pins import ALL_PINS

SRC_PATH = oracle_mod.__file__
with open(SRC_PATH, encoding="utf-8") as _f:
    SRC = _f.read()

MUTANTS = {
    "gqa_modulo_mapping": ("g = h // group\n        s = scale", "g = h % hkv\n        s = scale"),
    "causal_excludes_diagonal": ("np.arange(lk)[None, :] <= q_pos[:, None]",
                                 "np.arange(lk)[None, :] < q_pos[:, None]"),
    "scale_dropped": ("s = scale * (q[:, h, :] @ k[:, g, :].T)", "s = (q[:, h, :] @ k[:, g, :].T)"),
    "no_normalisation": ("        w /= w.sum(axis=1, keepdims=True)\n", ""),
    "values_from_keys": ("out[:, h, :] = w @ v[:, g, :]", "out[:, h, :] = w @ k[:, g, :]"),
    "gather_block_offset_swapped": ("physical = np.asarray(table_row)[p // block_size]\n    return cache[physical, p % block_size]",
                                    "physical = np.asarray(table_row)[p % block_size]\n    return cache[physical, p // block_size]"),
    "reshape_divmod_swapped": ("block, offset = divmod(s, block_size)",
                               "offset, block = divmod(s, block_size)"),
    "reshape_negative_slot_written": ("        if s < 0:\n            continue\n", ""),
    "decode_drops_current_token": ("return ref_contiguous_attention(q, k, v, scale, np.array([n - 1]))[0]",
                                   "return ref_contiguous_attention(q, k[:-1], v[:-1], scale, np.array([n - 2]))[0]"),
    "prefill_ignores_context_position": ("return ref_contiguous_attention(qr, k, v, scale, ctx_len + rows)",
                                         "return ref_contiguous_attention(qr, k, v, scale, rows)"),
    "merge_without_rescale": ("w = np.exp(ms - big_m)", "w = np.ones_like(ms)"),
    "partition_sum_without_exp": ("l[h] = e.sum()", "l[h] = float(len(e))"),
    "kv_bytes_without_k_and_v": ("return 2 * layers * kv_heads * head_dim * dtype_bytes",
                                 "return layers * kv_heads * head_dim * dtype_bytes"),
    "bf16_widened_wrong": ("(bits.astype(np.uint32) << 16)", "(bits.astype(np.uint32) << 15)"),
    "scale_kept_in_float64": ("return float(np.float32(scale))", "return float(scale)"),
    "copy_blocks_reversed": ("        kc[b] = k_cache[a]\n        vc[b] = v_cache[a]",
                             "        kc[a] = k_cache[b]\n        vc[a] = v_cache[b]"),
    "copy_blocks_v_from_k": ("        vc[b] = v_cache[a]", "        vc[b] = k_cache[a]"),
    "multi_query_positions_from_start": ("        pos = n - nq + np.arange(nq)\n", "        pos = np.arange(nq) + n - nq - 1\n"),
    "multi_query_no_causal_among_new": ("out[b, live] = ref_contiguous_attention(qb, k, v, scale, pos[live])",
                                        "out[b, live] = ref_contiguous_attention(qb, k, v, scale, np.full(len(live), n - 1))"),
}


def _load_mutant(old, new):
    assert SRC.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = SRC_PATH
    exec(compile(SRC.replace(old, new), SRC_PATH, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    mutant = _load_mutant(old, new)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except Exception as e:  # an assertion, or the mutant crashing on a pin's input
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutant {name}"


def test_unmutated_copy_passes_every_pin():
    mod = types.ModuleType("oracle_copy")
    exec(compile(SRC, SRC_PATH, "exec"), mod.__dict__)
    for pin in ALL_PINS:
        pin(mod)
