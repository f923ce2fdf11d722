"""Seeded synthetic inputs for the rotated W4A16 linear.

This module only draws random numbers and casts them to the storage dtypes. It
holds none of the method's arithmetic (no rotation, scaling, quantization or
matmul), so both the CPU oracle and the HIP path can take their inputs from it.

Recipe (the same for every workload):

* one ``numpy.random.SeedSequence(seed)`` per linear; its seven children, in
  order, drive ``x``, ``W``, the activation outlier channels, the weight outlier
  input columns, the stage pairings, the angles and the channel scales;
* ``x ~ N(0, 1)`` in float64, a fixed set of outlier channels multiplied by a
  factor in every row, then cast to float16;
* ``W ~ N(0, 0.02)`` in float64, a fixed set of outlier input columns
  multiplied by a factor, then cast to float16;
* stage k pairs channels by ``rng.permutation(D).reshape(D // 2, 2)``, so every
  channel is in exactly one pair of each stage;
* angles ``theta ~ U(-pi, pi)`` as float32, one per pair per stage;
* channel scales ``s = exp(N(0, 0.3))`` as float32 (positive).

The shapes follow the workloads the method is evaluated on: a tiny check case,
Qwen2.5-1.5B-shaped attention and MLP projections, and the seven linears of one
8B-class decoder layer (hidden 4096, MLP 14336, GQA kv dim 1024).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

GROUP = 128


@dataclasses.dataclass(frozen=True)
class LinearSpec:
    """One linear layer of a workload: y[M][N] = transform(x)[M][D] . W[N][D]^T."""

    name: str
    D: int
    N: int
    K: int
    x_outlier_frac: float = 0.005
    x_outlier_mult: float = 30.0
    w_outlier_frac: float = 0.01
    w_outlier_mult: float = 10.0
    x_outlier_chans: tuple = ()  # explicit channels (tiny case) instead of a fraction


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    linears: tuple  # of LinearSpec
    Ms: tuple  # token counts the workload is run at


def _tiny():
    return Workload(
        1,
        "tiny check 4x256->512 K=2",
        (LinearSpec("tiny", D=256, N=512, K=2, x_outlier_frac=0.0, x_outlier_mult=20.0,
                    w_outlier_frac=0.0, w_outlier_mult=1.0, x_outlier_chans=(3, 77)),),
        (4,),
    )


WORKLOADS = {
    1: _tiny(),
    2: Workload(
        2,
        "Qwen2.5-1.5B attention projections (q,k,v,o) decode",
        (LinearSpec("q", 1536, 1536, 8), LinearSpec("k", 1536, 256, 8),
         LinearSpec("v", 1536, 256, 8), LinearSpec("o", 1536, 1536, 8)),
        (1, 4, 16),
    ),
    3: Workload(
        3,
        "Qwen2.5-1.5B fused gate+up 1536->17920",
        (LinearSpec("gate_up", 1536, 17920, 8),),
        (1, 16, 256),
    ),
    4: Workload(
        4,
        "Qwen2.5-1.5B down_proj prefill 2048x8960->1536",
        (LinearSpec("down", 8960, 1536, 8),),
        (2048,),
    ),
    5: Workload(
        5,
        "8B-class decoder layer (7 linears)",
        (LinearSpec("q", 4096, 4096, 8), LinearSpec("k", 4096, 1024, 8),
         LinearSpec("v", 4096, 1024, 8), LinearSpec("o", 4096, 4096, 8),
         LinearSpec("gate", 4096, 14336, 8), LinearSpec("up", 4096, 14336, 8),
         LinearSpec("down", 14336, 4096, 8)),
        (64, 4096),
    ),
}


@dataclasses.dataclass
class LinearInputs:
    spec: LinearSpec
    x: np.ndarray  # float16 [M][D]
    W: np.ndarray  # float16 [N][D]
    pairs: np.ndarray  # int32 [K][D/2][2]
    theta: np.ndarray  # float32 [K][D/2]
    scale: np.ndarray  # float32 [D]


def _linear_seed(wid: int, index: int) -> np.random.SeedSequence:
    root = np.random.SeedSequence(wid)
    if len(WORKLOADS[wid].linears) == 1:
        return root
    return root.spawn(len(WORKLOADS[wid].linears))[index]


def _outlier_set(rng: np.random.Generator, D: int, frac: float) -> np.ndarray:
    count = int(round(frac * D))
    return np.sort(rng.choice(D, size=count, replace=False)) if count else np.zeros(0, np.int64)


def make_transform(kids, D: int, K: int):
    """Pairs, angles and scales from the last three of a linear's seven seed children."""
    r_pairs, r_theta, r_s = (np.random.default_rng(k) for k in kids[4:7])
    pairs = np.stack([r_pairs.permutation(D).reshape(D // 2, 2) for _ in range(K)]) if K else \
        np.zeros((0, D // 2, 2), np.int64)
    theta = r_theta.uniform(-math.pi, math.pi, size=(K, D // 2)).astype(np.float32)
    scale = np.exp(r_s.normal(0.0, 0.3, size=D)).astype(np.float32)
    return pairs.astype(np.int32), theta, scale


def make_linear(wid: int, index: int = 0, M: int | None = None, with_weights: bool = True,
                spec: LinearSpec | None = None, seed_seq: np.random.SeedSequence | None = None) -> LinearInputs:
    """Inputs of linear ``index`` of workload ``wid`` at ``M`` tokens.

    ``x`` is drawn at the workload's largest M and the first ``M`` rows are kept,
    so the smaller decode batches are prefixes of the larger ones.
    """
    if spec is None:
        wl = WORKLOADS[wid]
        spec = wl.linears[index]
        m_max = max(wl.Ms)
        ss = _linear_seed(wid, index)
    else:
        m_max = 1 if M is None else M
        ss = seed_seq
    kids = ss.spawn(7)
    r_x, r_w, r_xo, r_wo = (np.random.default_rng(k) for k in kids[:4])
    D, N = spec.D, spec.N
    M = m_max if M is None else M
    x = r_x.standard_normal((m_max, D))
    if spec.x_outlier_chans:
        xo = np.asarray(spec.x_outlier_chans, np.int64)
    else:
        xo = _outlier_set(r_xo, D, spec.x_outlier_frac)
    x[:, xo] *= spec.x_outlier_mult
    x = x[:M].astype(np.float16)
    if with_weights:
        W = r_w.normal(0.0, 0.02, size=(N, D))
        wo = _outlier_set(r_wo, D, spec.w_outlier_frac)
        W[:, wo] *= spec.w_outlier_mult
        W = W.astype(np.float16)
    else:
        W = np.zeros((0, D), np.float16)
    pairs, theta, scale = make_transform(kids, D, spec.K)
    return LinearInputs(spec, x, W, pairs, theta, scale)


# A Qwen2.5-1.5B-shaped decoder stack for whole-model decode and build measurements: 28 layers,
# each with q, k, v, o (hidden 1536, GQA kv dim 256), gate and up (1536 -> 8960) and down
# (8960 -> 1536), every linear with its own transform (K = 8).
MODEL_LAYERS = 28
MODEL_LINEARS = (LinearSpec("q", 1536, 1536, 8), LinearSpec("k", 1536, 256, 8),
                 LinearSpec("v", 1536, 256, 8), LinearSpec("o", 1536, 1536, 8),
                 LinearSpec("gate", 1536, 8960, 8), LinearSpec("up", 1536, 8960, 8),
                 LinearSpec("down", 8960, 1536, 8))
# the linears a decode step runs together: q/k/v read the same input, so do gate/up
MODEL_PHASES = ((0, 1, 2), (3,), (4, 5), (6,))


def make_model_linear(layer: int, index: int, M: int = 1, with_weights: bool = True) -> LinearInputs:
    """Linear ``index`` of decoder layer ``layer`` of the 1.5B-shaped stack (seed: [6, layer])."""
    ss = np.random.SeedSequence([6, layer]).spawn(len(MODEL_LINEARS))[index]
    return make_linear(0, spec=MODEL_LINEARS[index], seed_seq=ss, M=M, with_weights=with_weights)


def custom_linear(seed: int, M: int, D: int, N: int, K: int, x_outlier_frac=0.005,
                  w_outlier_frac=0.01) -> LinearInputs:
    """Inputs with the same distributions at arbitrary shapes (ragged tails, edge cases)."""
    spec = LinearSpec(f"custom{seed}", D, N, K, x_outlier_frac=x_outlier_frac,
                      w_outlier_frac=w_outlier_frac)
    return make_linear(0, spec=spec, seed_seq=np.random.SeedSequence([seed, M, D, N, K]), M=M)


def algorithmic_bytes(M: int, D: int, N: int, K: int, out_bytes: int = 2) -> int:
    """Bytes the fused rotated linear must move: packed weights, fp16 scale and zero
    per 128-group, x in, y out, and the transform's parameters -- per stage one int16
    pair index per channel and one fp32 angle per pair (4 K D bytes), and one fp32
    channel scale per channel (4 D bytes)."""
    w = N * D // 2 + N * (D // GROUP) * 4
    return w + 2 * M * D + out_bytes * M * N + 4 * K * D + 4 * D


def transform_bytes(M: int, D: int, K: int) -> int:
    """Bytes the standalone transform must move: x in, x' out (fp16) and the transform's
    parameters as in ``algorithmic_bytes``."""
    return 4 * M * D + 4 * K * D + 4 * D


def plain_bytes(M: int, D: int, N: int, out_bytes: int = 2) -> int:
    """Bytes of the plain W4A16 linear (no transform parameters)."""
    return N * D // 2 + N * (D // GROUP) * 4 + 2 * M * D + out_bytes * M * N


# The library's packed-weight layout, written out from its definition in include/paro.h ("Packed
# weights"): rows in blocks of 16 (the last block holds the N % 16 remaining rows), block b
# starting at byte 16 b D/2 and holding group g (64 bytes per row) of its R_b rows contiguously,
# row r of the block at byte 16 b D/2 + g R_b 64 + r 64. The oracle packs row-major [N][D/2];
# these move a host array between the two orders (the bytes are the same).
def qweight_to_blocked(q):
    q = np.asarray(q, np.uint8)
    N, H = q.shape
    out = np.empty(N * H, np.uint8)
    for b0 in range(0, N, 16):
        R = min(16, N - b0)
        out[b0 * H:(b0 + R) * H] = q[b0:b0 + R].reshape(R, H // 64, 64).transpose(1, 0, 2).reshape(-1)
    return out.reshape(N, H)


def qweight_from_blocked(qb):
    qb = np.asarray(qb, np.uint8)
    N, H = qb.shape
    flat = qb.reshape(-1)
    out = np.empty((N, H), np.uint8)
    for b0 in range(0, N, 16):
        R = min(16, N - b0)
        out[b0:b0 + R] = flat[b0 * H:(b0 + R) * H].reshape(H // 64, R, 64).transpose(1, 0, 2).reshape(R, H)
    return out
