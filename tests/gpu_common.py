"""Helpers shared by the GPU parity tests: device transfer, oracle caching, tolerances.

Expected values come only from ``oracle/`` (CPU, float64) applied to the seeded
inputs of ``workloads``; nothing the HIP path computes is fed back to the oracle.
"""
from __future__ import annotations

import functools
import sys

import numpy as np

import oracle as O
import workloads as W


def log(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


# the library's blocked qweight order <-> the oracle's row-major one (include/paro.h)
to_blocked = W.qweight_to_blocked
from_blocked = W.qweight_from_blocked


def dev_weights(w, torch):
    """Oracle-packed (row-major qweight, scales, zeros) -> the library's device operands."""
    qw, sc, z = w
    return dev(to_blocked(qw), torch), dev(sc, torch), dev(z, torch)


def host_weights(w):
    """The library's device (qweight, scales, zeros) -> host arrays with a row-major qweight."""
    qw, sc, z = w
    return from_blocked(host(qw)), host(sc), host(z)


@functools.lru_cache(maxsize=None)
def linear_inputs(wid: int, index: int):
    return W.make_linear(wid, index)


def sample_rows(n_total: int, n_pick: int, seed: int) -> np.ndarray:
    if n_total <= n_pick:
        return np.arange(n_total)
    rng = np.random.default_rng(seed)
    picks = rng.choice(n_total, size=n_pick - 2, replace=False)
    return np.unique(np.concatenate([picks, [0, n_total - 1]]))  # always include the ragged ends


@functools.lru_cache(maxsize=None)
def oracle_pack_rows(wid: int, index: int, rows_key: tuple | None):
    """Oracle pack of selected weight rows (None = all rows). Rows are independent."""
    L = linear_inputs(wid, index)
    Wm = L.W if rows_key is None else L.W[np.asarray(rows_key)]
    return O.pack_weights(Wm, L.pairs, L.theta, L.scale)


def ulp16(a: np.ndarray) -> np.ndarray:
    """Spacing of float16 numbers at |a| (normal range; subnormal spacing below 2^-14)."""
    a = np.abs(np.asarray(a, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def rotate_bound(a64: np.ndarray, x64: np.ndarray, scale: np.ndarray, K: int) -> np.ndarray:
    """Per-element bound for the float32 transform rounded to float16 against the float64
    oracle ``a64``. Each float32 stage moves an element by at most a few 2^-24 of its pair's
    norm, which never exceeds the row's 2-norm ||x|| (the rotations preserve it); the final
    multiply by the float32 1/s adds two more roundings. So the float32 value v satisfies
    |v - a| <= delta = (K + 2) * 4 * 2^-24 * ||x|| / s, and rounding v to float16 adds at
    most half a float16 ulp at |a| + delta."""
    rownorm = np.linalg.norm(x64, axis=1, keepdims=True)
    delta = (K + 2) * 4.0 * 2.0 ** -24 * rownorm / np.asarray(scale, np.float64)[None, :]
    return 0.5 * ulp16(np.abs(a64) + delta) + delta


def rotate_off_cap(n: int, K: int) -> int:
    """Most elements of n that may differ from the float16 rounding of the float64 transform: the
    kernel's float32 result lands on the other side of a float16 rounding boundary now and then.
    Emulating its float32 sequence on the CPU puts 0.04-0.07% of elements off at K = 8 and 0.19%
    at K = 64 (about 3e-5 per stage); the cap is 2e-4 per stage (plus two for the final scaling),
    and at least 4 elements."""
    return max(4, int(2e-4 * (K + 2) * n))


def masked_max_abs(got: np.ndarray, ref: np.ndarray, below: float) -> float:
    """Max |got - ref| over the outputs with |ref| < below (0 if there are none)."""
    m = np.abs(ref) < below
    return float(np.abs(got.astype(np.float64) - ref)[m].max()) if m.any() else 0.0


def fp16_path_bound(a: np.ndarray, deq: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-output bound on |y16 - a . deq^T| for the float16 output of the rotated linear, where a is
    the float64 transform and ref = a . deq^T. Three terms: rounding x' once to float16 moves each
    output by at most e_x = |f16(a) - a| . |deq|^T (exact worst case, triangle inequality); the
    float32 sums of exact products add at most e_acc = (128 + G + 4) 2^-24 |f16(a)| . |deq|^T (up to
    128 additions inside a group, G = D/128 across groups, the scale multiplies); rounding the result
    to float16 adds half a float16 spacing at |ref| + e_x + e_acc."""
    a16 = f16_of(a)
    G = a.shape[1] // 128
    e_x = np.abs(a16 - a) @ np.abs(deq).T
    e_acc = (128 + G + 4) * 2.0 ** -24 * (np.abs(a16) @ np.abs(deq).T)
    return e_x + e_acc + 0.5 * ulp16(np.abs(ref) + e_x + e_acc)


def over_bound(err: np.ndarray, bound: np.ndarray) -> float:
    """max(err / bound), counting 0 / 0 as 0 (zero weight rows give zero error and bound) and any
    error where the bound is 0 as infinite."""
    err = np.abs(err)
    r = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    return float(r.max()) if r.size else 0.0


def f16_of(a: np.ndarray) -> np.ndarray:
    return O.f16_rne(a).astype(np.float64)


def linear_metrics(got: np.ndarray, ref: np.ndarray):
    err = np.abs(got.astype(np.float64) - ref)
    return float(err.max()), float(np.linalg.norm(got.astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-30))


# The linear bar: max-abs <= 1e-2 and relative L2 <= 2e-3 against the oracle applied to the
# same dequantized weights (and, for the rotated linear, the same float16 activations).
MAX_ABS = 1e-2
REL_L2 = 2e-3
