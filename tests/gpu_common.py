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


def linear_metrics(got: np.ndarray, ref: np.ndarray):
    err = np.abs(got.astype(np.float64) - ref)
    return float(err.max()), float(np.linalg.norm(got.astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-30))


# The linear bar: max-abs <= 1e-2 and relative L2 <= 2e-3 against the oracle applied to the
# same dequantized weights (and, for the rotated linear, the same float16 activations).
MAX_ABS = 1e-2
REL_L2 = 2e-3
