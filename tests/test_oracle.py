"""The CPU oracle against its pins, and the pins against planted mistakes."""
import importlib.util
import os
import types

import numpy as np
import pytest

import oracle
import oracle_pins as P

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "flce_oracle.py")


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)


# Each mutation is a plausible mistake: a dropped term, a wrong sign or
# index, a missing stabiliser, an overwrite instead of an accumulation.
MUTATIONS = {
    "dropped_onehot": ("P[rows, target[rows]] -= 1.0", "P[rows, target[rows]] -= 0.0"),
    "onehot_sign": ("P[rows, target[rows]] -= 1.0", "P[rows, target[rows]] += 1.0"),
    "no_row_max": ("M = Z.max(axis=1)\n", "M = 0.0 * Z.max(axis=1)\n"),
    "lse_drops_max": ("return M + np.log(", "return np.log("),
    "unnormalised_softmax": ("P = np.exp(Z - lse[:, None])",
                             "P = np.exp(Z - Z.max(axis=1)[:, None])"),
    "ignored_rows_kept": ("P[~valid] = 0.0", "pass"),
    "dropped_grad_scale": ("return grad_scale * P", "return P"),
    "loss_sign": ("loss[r0 + idx] = l[idx] - Z[idx, tg[idx]]",
                  "loss[r0 + idx] = Z[idx, tg[idx]] - l[idx]"),
    "target_off_by_one": ("zt = Z[idx, target[r0:r1][idx]]",
                          "zt = Z[idx, target[r0:r1][idx] - 1]"),
    "gather_off_by_one": ("l[idx] - Z[idx, tg[idx]]", "l[idx] - Z[idx, tg[idx] - 1]"),
    "dH_sign": ("dH[r0:r1] = dZ @ W", "dH[r0:r1] = -(dZ @ W)"),
    "dW_overwrite": ("dW += dZ.T @ H[r0:r1]", "dW = dZ.T @ H[r0:r1]"),
    "dW_wrong_operand": ("dW += dZ.T @ H[r0:r1]", "dW += dZ.T @ H[r0:r1][::-1]"),
    "range_check": ("bad = valid & ((target < 0) | (target >= V))", "bad = valid & (target < 0)"),
    "backward_swapped": ("    return dH, dW\n", "    return dW, dH\n"),
    "backward_drops_scale": ("ignore_index, grad_scale, row_chunk)\n    return dH, dW",
                             "ignore_index, 1.0, row_chunk)\n    return dH, dW"),
}


def _mutant(name):
    src = open(ORACLE_SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mod = types.ModuleType("flce_oracle_mutant_" + name)
    exec(compile(src.replace(old, new), ORACLE_SRC + ":" + name, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant(name)
    caught = []
    with np.errstate(all="ignore"):
        for pin in P.ALL_PINS:
            try:
                pin(mod)
            except Exception as e:  # AssertionError, IndexError, ...
                caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin fails for the planted mistake {name}"
