"""CPU oracle for the ParoQuant rotated W4A16 linear -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module. The product path (the HIP library and its
Python binding) never imports, calls or links it, and this module imports
nothing from the product path.

Everything is plain NumPy in float64, written to be checked by eye against the
pages it follows (cited per function):

* "ParoQuant: pairwise rotations that survive deployment" (hungho77.github.io),
  sections "A rotation small enough to execute" (the 2x2 Givens equation, the
  disjoint pairs, stages, channel-wise scaling, the build-time fold and the
  runtime inverse activation-side transform), "My reduced-calibration
  experiment" (INT4, group size 128) and "From fake quantization to a real
  TensorRT engine" (one rotation operator plus one group-wise INT4 GEMM
  operator per linear; real INT4 packing).
* The arXiv abstract of "ParoQuant: Pairwise Rotation Quantization for
  Efficient Reasoning LLM Inference" (mlsanity.com paper card): independent
  Givens rotations with channel-wise scaling, weight-only quantization.

Readings taken where the pages leave a step open (all listed in the design
notes): the first index i of a stored pair takes +sin(theta); stage 1 is applied
first on both sides; the weights are multiplied by s and the activations divided
by s; cos/sin are rounded once to float32 from float64; the INT4 quantizer is the
min/max asymmetric one with the scale rounded to float16 and an integer
zero-point 0..15; packing is row-major [N][D/2] with the even channel in the low
nibble; scales and zeros are float16 [N][D/128].

Parity status: every function here is pinned by a CPU test against closed forms,
brute force or invariants (see tests/test_oracle_pins.py). The sign convention
linking theta to the inverse transform (theta versus -theta with the stage order
reversed) is the one reading no printed value pins; it changes no result, since
weights and activations use the same convention.
"""
from __future__ import annotations

import math

import numpy as np

GROUP = 128  # "INT4 and group size 128" (section "My reduced-calibration experiment")
QMAX = 15  # INT4 asymmetric: codes 0..15
SCALE_FLOOR = 1e-5


# --------------------------------------------------------------------------- #
# Pairings, angles, scales
# --------------------------------------------------------------------------- #

def check_stage_pairs(pairs: np.ndarray, D: int) -> None:
    """Every stage must pair each of the D channels exactly once.

    The page ("A rotation small enough to execute") requires that no channel
    appears in two rotations of one stage; with D/2 pairs per stage that is the
    same as every channel appearing exactly once.
    """
    pairs = np.asarray(pairs)
    if D % 2:
        raise ValueError("D must be even")
    if pairs.ndim != 3 or pairs.shape[1:] != (D // 2, 2):
        raise ValueError(f"pairs must be [K][{D // 2}][2], got {pairs.shape}")
    for k in range(pairs.shape[0]):
        seen = np.sort(pairs[k].ravel())
        if not np.array_equal(seen, np.arange(D)):
            raise ValueError(f"stage {k} is not a perfect matching of 0..{D - 1}")


def stage_cos_sin(theta: np.ndarray):
    """cos and sin of every angle, evaluated in float64 by the C library and
    rounded once to float32, returned as float64 arrays.

    The pages give one learned angle per pair (the 2x2 equation of "A rotation
    small enough to execute"); the storage precision is our reading.
    """
    th = np.asarray(theta, np.float32)
    c = np.empty(th.shape, np.float64)
    s = np.empty(th.shape, np.float64)
    flat_t, flat_c, flat_s = th.ravel(), c.reshape(-1), s.reshape(-1)
    for n in range(flat_t.size):
        t = float(flat_t[n])
        flat_c[n] = float(np.float32(math.cos(t)))
        flat_s[n] = float(np.float32(math.sin(t)))
    return c, s


def f16_rne(a: np.ndarray) -> np.ndarray:
    """float64 -> float16, one round-to-nearest-even step (NumPy's direct
    double-to-half conversion; pinned against exhaustive search in the tests)."""
    return np.asarray(a, np.float64).astype(np.float16)


# --------------------------------------------------------------------------- #
# The transform (Givens stages + channel-wise scaling)
# --------------------------------------------------------------------------- #

def givens_stages(v: np.ndarray, pairs: np.ndarray, c: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Apply the K stages to the last axis of ``v`` (float64), stage 1 first.

    For each pair (i, j) of a stage, with c = cos(theta), s = sin(theta):
        v_i <- c*v_i + s*v_j
        v_j <- -s*v_i + c*v_j      (written c*v_j - s*v_i)
    both from the values before the update: the 2x2 equation of
    "A rotation small enough to execute". The pairs of one stage are disjoint,
    so updating them all at once equals updating them one by one.
    """
    out = np.array(v, np.float64, copy=True)
    for k in range(pairs.shape[0]):
        i = pairs[k, :, 0]
        j = pairs[k, :, 1]
        vi = out[..., i].copy()
        vj = out[..., j].copy()
        ck, sk = c[k], s[k]
        out[..., i] = ck * vi + sk * vj
        out[..., j] = ck * vj - sk * vi
    return out


def givens_stages_inverse(v: np.ndarray, pairs: np.ndarray, c: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Undo ``givens_stages``: stages K..1, each with the transposed 2x2 matrix."""
    out = np.array(v, np.float64, copy=True)
    for k in reversed(range(pairs.shape[0])):
        i = pairs[k, :, 0]
        j = pairs[k, :, 1]
        vi = out[..., i].copy()
        vj = out[..., j].copy()
        ck, sk = c[k], s[k]
        out[..., i] = ck * vi - sk * vj
        out[..., j] = sk * vi + ck * vj
    return out


def transform_activations(x: np.ndarray, pairs, theta, scale) -> np.ndarray:
    """Runtime activation-side transform: the Givens stages, then divide by s.

    "Channel-wise scaling follows the rotations" and, at runtime, "the inverse
    activation-side transformation is executed immediately before the packed
    INT4 linear" (section "A rotation small enough to execute"). With weight rows
    mapped to S.G.w (S = diag(s), G = G_K...G_1 orthogonal), keeping x.w
    unchanged needs x -> S^-1.G.x: the same stages in the same order, then 1/s.
    """
    c, s = stage_cos_sin(theta)
    a = givens_stages(np.asarray(x, np.float64), pairs, c, s)
    return a / np.asarray(scale, np.float64)


def untransform_activations(a: np.ndarray, pairs, theta, scale) -> np.ndarray:
    """Inverse of ``transform_activations``: multiply by s, then undo the stages."""
    c, s = stage_cos_sin(theta)
    return givens_stages_inverse(np.asarray(a, np.float64) * np.asarray(scale, np.float64), pairs, c, s)


def fold_weights(W: np.ndarray, pairs, theta, scale) -> np.ndarray:
    """Build-time weight-side transform ("weight transformations are folded",
    section "A rotation small enough to execute"): every row of W goes through
    the same stages along D, then is multiplied by s. Float64, products then a
    single add or subtract per output, as in ``givens_stages``."""
    c, s = stage_cos_sin(theta)
    b = givens_stages(np.asarray(W, np.float64), pairs, c, s)
    return b * np.asarray(scale, np.float64)


# --------------------------------------------------------------------------- #
# Group-wise asymmetric INT4 quantization and packing
# --------------------------------------------------------------------------- #

def quantize_groups(b: np.ndarray):
    """Asymmetric INT4 quantization of each 128-wide group along D.

    Per (row n, group g), in float64:
        lo, hi   = min, max of the group
        scale16  = float16(max((hi - lo) / 15, 1e-5))        (one RNE rounding)
        z        = clip(rint(-lo / scale16), 0, 15)
        q        = clip(rint(b / scale16) + z, 0, 15)
    rint rounds half to even. Returns q (uint8 [N][D]), scales (float16
    [N][D/128]) and zeros (float16 [N][D/128], integers 0..15).
    Group size 128 and INT4: section "My reduced-calibration experiment"; the
    quantizer itself is the textbook min/max one (our reading).
    """
    b = np.asarray(b, np.float64)
    N, D = b.shape
    if D % GROUP:
        raise ValueError("D must be a multiple of 128")
    G = D // GROUP
    bg = b.reshape(N, G, GROUP)
    lo = bg.min(axis=2)
    hi = bg.max(axis=2)
    step = np.maximum((hi - lo) / QMAX, SCALE_FLOOR)
    scale16 = f16_rne(step)
    sc = scale16.astype(np.float64)
    z = np.clip(np.rint(-lo / sc), 0, QMAX)
    q = np.clip(np.rint(bg / sc[:, :, None]) + z[:, :, None], 0, QMAX)
    return q.reshape(N, D).astype(np.uint8), scale16, z.astype(np.float16)


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte, row-major: byte t of row n holds channel 2t in
    bits 0..3 and channel 2t+1 in bits 4..7 ("real INT4 packing", section
    "From fake quantization to a real TensorRT engine"; the layout is ours)."""
    q = np.asarray(q, np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(qweight: np.ndarray) -> np.ndarray:
    qw = np.asarray(qweight, np.uint8)
    N, half = qw.shape
    q = np.empty((N, 2 * half), np.uint8)
    q[:, 0::2] = qw & 0xF
    q[:, 1::2] = qw >> 4
    return q


def pack_weights(W: np.ndarray, pairs, theta, scale):
    """Build-time path: fold the transform into W, quantize per group, pack.
    Returns (qweight uint8 [N][D/2], scales float16 [N][D/128], zeros float16 [N][D/128])."""
    b = fold_weights(W, pairs, theta, scale)
    q, sc, z = quantize_groups(b)
    return pack_nibbles(q), sc, z


def dequantize(qweight, scales, zeros) -> np.ndarray:
    """(q - z) * scale in float64 (exact: at most 15 significant bits)."""
    q = unpack_nibbles(qweight).astype(np.float64)
    N, D = q.shape
    G = D // GROUP
    sc = np.asarray(scales, np.float64).reshape(N, G, 1)
    z = np.asarray(zeros, np.float64).reshape(N, G, 1)
    return ((q.reshape(N, G, GROUP) - z) * sc).reshape(N, D)


# --------------------------------------------------------------------------- #
# Linears
# --------------------------------------------------------------------------- #

def w4a16_linear(x: np.ndarray, qweight, scales, zeros) -> np.ndarray:
    """Plain group-wise INT4 weight-only linear: y = x . deq^T in float64."""
    return np.asarray(x, np.float64) @ dequantize(qweight, scales, zeros).T


def rotated_linear(x: np.ndarray, pairs, theta, scale, qweight, scales, zeros,
                   round_activations: bool = False) -> np.ndarray:
    """Transform the activations, then the INT4 linear (section "A rotation small
    enough to execute": the inverse activation-side transform runs immediately
    before the packed INT4 linear). With ``round_activations`` the transformed
    activations are rounded to float16 first -- the 16-bit operand the GEMM of a
    W4A16 linear consumes."""
    a = transform_activations(x, pairs, theta, scale)
    if round_activations:
        a = f16_rne(a).astype(np.float64)
    return a @ dequantize(qweight, scales, zeros).T


def rotate_f16(x: np.ndarray, pairs, theta, scale) -> np.ndarray:
    """The standalone rotate call's result: the activation transform rounded once to float16."""
    return f16_rne(transform_activations(x, pairs, theta, scale))
