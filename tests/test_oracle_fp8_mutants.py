"""Plant plausible mistakes in copies of the FP8 oracle and check a pin catches each."""

import types

import pytest

import oracle.kv_fp8 as fp8_mod
from oracle_pins_fp8 import FP8_PINS

SRC_PATH = fp8_mod.__file__
with open(SRC_PATH, encoding="utf-8") as _f:
    SRC = _f.read()

MUTANTS = {
    "exponent_bias_8": ("normal = np.ldexp(1.0 + m / 8.0, e - 7)", "normal = np.ldexp(1.0 + m / 8.0, e - 8)"),
    "subnormal_without_min_exponent": ("sub = np.ldexp(m / 8.0, _MIN_NORMAL_EXP)", "sub = np.ldexp(m / 8.0, -7)"),
    "round_half_up": ("steps = np.rint(np.ldexp(a, -step))", "steps = np.floor(np.ldexp(a, -step) + 0.5)"),
    "truncate": ("steps = np.rint(np.ldexp(a, -step))", "steps = np.floor(np.ldexp(a, -step))"),
    "no_saturation": ("a = np.minimum(np.abs(x), E4M3_MAX)", "a = np.abs(x)"),
    "four_mantissa_steps": ("e - 1 - 3)", "e - 1 - 2)"),
    "scale_for_240": ("amax / np.float32(E4M3_MAX)", "amax / np.float32(240.0)"),
    "quotient_in_float64": ("y = (x / scale[..., None]).astype(np.float32)",
                            "y = x.astype(np.float64) / scale[..., None]"),
    "scale_not_applied": ("return e4m3_to_float64(codes) * np.asarray(scales, np.float32).astype(np.float64)[..., None]",
                          "return e4m3_to_float64(codes)"),
    "scales_at_head_slot": ("ksc[block, :, offset] = ks[t]", "ksc[block, :, offset % ksc.shape[2]] = ks[t][::-1]"),
    "gather_scales_offset_swapped": ("return scales[physical, :, p % block_size]",
                                     "return scales[physical, :, (p // block_size) % block_size]"),
    "v_dequantised_with_k_scales": ("v = _dequantized_tokens(v_cache, v_scales, block_tables[b], n)",
                                    "v = _dequantized_tokens(v_cache, k_scales, block_tables[b], n)"),
    "prefill_k_with_v_scales": ("k = _dequantized_tokens(k_cache, k_scales, table_row, n)",
                                "k = _dequantized_tokens(k_cache, v_scales, table_row, n)"),
    "negative_slot_written": ("        if s < 0:\n            continue\n", ""),
}


def _load(src):
    mod = types.ModuleType("oracle.kv_fp8_mutant")
    mod.__file__ = SRC_PATH
    mod.__package__ = "oracle"
    exec(compile(src, SRC_PATH, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fp8_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mutant = _load(SRC.replace(old, new))
    caught = []
    for pin in FP8_PINS:
        try:
            pin(mutant)
        except Exception as e:  # an assertion, or the mutant crashing on a pin's input
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutant {name}"


def test_unmutated_fp8_copy_passes_every_pin():
    mod = _load(SRC)
    for pin in FP8_PINS:
        pin(mod)
