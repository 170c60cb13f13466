"""Planted mistakes in copies of the CPU oracle must each fail a pin.

Each mutant is the oracle's source with one plausible error substituted
(a dropped term, a wrong index or sign, an off-by-one mask, a transposed
operand).  A mutant that passes every pin would mean the pins cannot tell
that mistake from the definition.  Runs on the CPU only.
"""

import os
import types

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC_PATH = os.path.join(os.path.dirname(oracle.__file__), "attention.py")

MUTANTS = {
    "gather_ignores_table": (
        "dense[start:start + take] = cache[int(table_row[j]), :take]",
        "dense[start:start + take] = cache[j, :take]"),
    "gather_wrong_block_order": (
        "for j in range(-(-n // block_size)):\n        start = j * block_size",
        "for j in range(-(-n // block_size)):\n        start = (-(-n // block_size) - 1 - j) * block_size"),
    "gqa_modulo_mapping": (
        "g = h // group",
        "g = h % Hkv"),
    "mask_excludes_self": (
        "visible = np.arange(n)[None, :] <= np.asarray(query_pos)[:, None]",
        "visible = np.arange(n)[None, :] < np.asarray(query_pos)[:, None]"),
    "mask_ignored_for_exp": (
        "e = np.where(visible[t], np.exp(scores[t] - m), acc_dtype(0))",
        "e = np.exp(np.where(visible[t], scores[t], 0) - m)"),
    "normalise_by_max": (
        "weights[t] = e / e.sum()",
        "weights[t] = e / e.max()"),
    "softmax_sign_flip": (
        "np.exp(scores[t] - m)",
        "np.exp(m - scores[t])"),
    "scale_dropped": (
        "scores = (q_h @ k_g.T) * acc_dtype(scale)",
        "scores = (q_h @ k_g.T) * acc_dtype(1.0)"),
    "scale_squared": (
        "scores = (q_h @ k_g.T) * acc_dtype(scale)",
        "scores = (q_h @ k_g.T) * acc_dtype(scale) * acc_dtype(scale)"),
    "values_are_keys": (
        "out[:, h, :] = weights @ np.asarray(v[:, g, :], dtype=acc_dtype)",
        "out[:, h, :] = weights @ np.asarray(k[:, g, :], dtype=acc_dtype)"),
    "decode_excludes_newest": (
        "np.array([n - 1]), acc_dtype)",
        "np.array([n - 2]), acc_dtype)"),
    "prefill_top_left_causal": (
        "positions = n - q_len + np.arange(q_len)",
        "positions = np.arange(q_len)"),
    "prefill_off_by_one": (
        "positions = n - q_len + np.arange(q_len)",
        "positions = n - q_len + np.arange(q_len) - 1"),
    "write_block_offset_swapped": (
        "block_id = slot // block_size\n        offset = slot % block_size",
        "block_id = slot % block_size\n        offset = slot // block_size"),
    "write_ignores_skip": (
        "if slot < 0:\n            continue",
        "if slot < -1:\n            continue"),
    "write_value_into_key": (
        "v[block_id, offset] = value[t]",
        "v[block_id, offset] = key[t]"),
    "write_in_place": (
        "k = np.array(k_cache, copy=True)",
        "k = k_cache"),
    "decode_output_width_from_key": (
        "out = np.zeros((S, Hq, v_cache.shape[3]), dtype=acc_dtype)",
        "out = np.zeros((S, Hq, D), dtype=acc_dtype)"),
    "no_guard_for_rows_without_keys": (
        "if not visible[t].any():",
        "if False:"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC_PATH).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    src = src.replace(old, new, 1)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or the mutant crashing
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches mutant {name}"
