"""CPU tests: the oracle against its pins, and broken copies of the oracle against them."""
import importlib.util
import os
import sys
import types

import pytest

import oracle
from tests import oracle_pins as P

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "paro_oracle.py")


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)


# Plausible slips, each planted in a copy of the oracle's source on the CPU.
MUTANTS = {
    "sin sign flipped": ("out[..., i] = ck * vi + sk * vj", "out[..., i] = ck * vi - sk * vj"),
    "dropped cross term": ("out[..., j] = ck * vj - sk * vi", "out[..., j] = ck * vj"),
    "pair roles swapped": ("i = pairs[k, :, 0]\n        j = pairs[k, :, 1]\n        vi = out[..., i].copy()\n        vj = out[..., j].copy()\n        ck, sk = c[k], s[k]\n        out[..., i] = ck * vi + sk * vj",
                           "i = pairs[k, :, 1]\n        j = pairs[k, :, 0]\n        vi = out[..., i].copy()\n        vj = out[..., j].copy()\n        ck, sk = c[k], s[k]\n        out[..., i] = ck * vi + sk * vj"),
    "stages reversed": ("    for k in range(pairs.shape[0]):\n        i = pairs[k, :, 0]",
                        "    for k in reversed(range(pairs.shape[0])):\n        i = pairs[k, :, 0]"),
    "in-place update (stale vi)": ("out[..., j] = ck * vj - sk * vi", "out[..., j] = ck * vj - sk * out[..., i]"),
    "activation multiplies by s": ("return a / np.asarray(scale, np.float64)", "return a * np.asarray(scale, np.float64)"),
    "weights divide by s": ("return b * np.asarray(scale, np.float64)", "return b / np.asarray(scale, np.float64)"),
    "cos/sin kept in float64": ("flat_c[n] = float(np.float32(math.cos(t)))", "flat_c[n] = math.cos(t)"),
    "zero-point sign": ("z = np.clip(np.rint(-lo / sc), 0, QMAX)", "z = np.clip(np.rint(lo / sc), 0, QMAX)"),
    "scale not rounded to fp16": ("sc = scale16.astype(np.float64)", "sc = step"),
    "round half up": ("q = np.clip(np.rint(bg / sc[:, :, None]) + z[:, :, None], 0, QMAX)",
                      "q = np.clip(np.floor(bg / sc[:, :, None] + 0.5) + z[:, :, None], 0, QMAX)"),
    "range divided by 16": ("step = np.maximum((hi - lo) / QMAX, SCALE_FLOOR)", "step = np.maximum((hi - lo) / 16, SCALE_FLOOR)"),
    "nibble order swapped": ("return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)",
                             "return (q[:, 1::2] | (q[:, 0::2] << 4)).astype(np.uint8)"),
    "dequant forgets zero": ("return ((q.reshape(N, G, GROUP) - z) * sc).reshape(N, D)",
                             "return (q.reshape(N, G, GROUP) * sc).reshape(N, D)"),
    "contraction index misaligned": ("return np.asarray(x, np.float64) @ dequantize(qweight, scales, zeros).T",
                                     "return np.asarray(x, np.float64)[:, ::-1] @ dequantize(qweight, scales, zeros).T"),
    "f16 via float32 (double rounding)": ("return np.asarray(a, np.float64).astype(np.float16)",
                                          "return np.asarray(a, np.float64).astype(np.float32).astype(np.float16)"),
    "matching check skipped": ("        if not np.array_equal(seen, np.arange(D)):", "        if False:"),
}


def _mutant(name, old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation '{name}' does not apply exactly once"
    mod = types.ModuleType(f"oracle_mutant")
    exec(compile(src.replace(old, new), ORACLE_SRC + f"[{name}]", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mod = _mutant(name, *MUTANTS[name])
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted slip '{name}'"
