"""Pins that tie the CPU oracle to what the pages and the mathematics fix.

Each ``pin_*`` takes an oracle module ``o`` and raises AssertionError when the
oracle disagrees with something other than itself: the 2x2 Givens equation and
the stage semantics of "ParoQuant: pairwise rotations that survive deployment"
(section "A rotation small enough to execute"), hand-worked examples under
``tests/golden/``, dense-matrix brute force, invariants (pair norms, x.W^T
invariance, forward-then-inverse), closed-form quantizer groups, exhaustive
float16 rounding and pure-Python loops on tiny inputs.

``tests/test_oracle_pins.py`` runs them against the oracle (all must pass) and
against deliberately broken copies of the oracle (each copy must fail at least
one), which shows that a plausible slip in the oracle cannot pass unnoticed.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _random_transform(rng, D, K):
    pairs = np.stack([rng.permutation(D).reshape(D // 2, 2) for _ in range(K)]).astype(np.int32) \
        if K else np.zeros((0, D // 2, 2), np.int32)
    theta = rng.uniform(-math.pi, math.pi, (K, D // 2)).astype(np.float32)
    scale = np.exp(rng.normal(0, 0.3, D)).astype(np.float32)
    return pairs, theta, scale


# ----------------------------------------------------------------------------- #
# float16 rounding
# ----------------------------------------------------------------------------- #

def _all_f16_sorted():
    bits = np.arange(0, 0x7C00, dtype=np.uint16)  # +0 .. largest finite
    pos = bits.view(np.float16).astype(np.float64)
    return pos, bits


def _nearest_even_f16(v: float):
    """Exhaustive-search round-to-nearest-even of a float64 into float16 (finite range)."""
    pos, bits = _all_f16_sorted()
    a = abs(v)
    k = int(np.searchsorted(pos, a))
    cands = [c for c in (k - 1, k) if 0 <= c < len(pos)]
    fa = Fraction(a)
    best = min(cands, key=lambda c: (abs(Fraction(pos[c]) - fa), int(bits[c]) & 1))
    r = pos[best]
    return -r if v < 0 else r


def pin_f16_rounding(o):
    rng = _rng(11)
    pos, _ = _all_f16_sorted()
    mids = (pos[:-1] + pos[1:]) / 2  # exact ties (float64 holds them)
    probes = np.concatenate([
        mids[::97], np.nextafter(mids[::89], 0), np.nextafter(mids[::83], 1),
        rng.normal(0, 1, 300) * 10.0 ** rng.integers(-7, 4, 300),
        np.array([1e-5, 6.1e-5, 2 / 15, 0.1, 65504.0, 1 / 3]),
    ])
    probes = probes[np.abs(probes) < 65504]
    got = o.f16_rne(probes).astype(np.float64)
    for v, g in zip(probes, got):
        e = _nearest_even_f16(float(v))
        assert g == e, f"f16 rounding of {v!r}: got {g!r}, want {e!r}"


# ----------------------------------------------------------------------------- #
# Givens rotation and stages
# ----------------------------------------------------------------------------- #

def pin_givens_closed_form(o):
    """The printed 2x2 equation: (1,0) -> (cos, -sin), (0,1) -> (sin, cos) for pair (i, j)."""
    for t in (0.7, -2.3, 3.0):
        c = float(np.float32(math.cos(float(np.float32(t)))))
        s = float(np.float32(math.sin(float(np.float32(t)))))
        pairs = np.array([[[0, 1]]], np.int32)
        theta = np.array([[t]], np.float32)
        one = np.ones(2, np.float32)
        a = o.transform_activations(np.array([[1.0, 0.0], [0.0, 1.0]]), pairs, theta, one)
        assert a[0, 0] == c and a[0, 1] == -s, (t, a[0], c, s)
        assert a[1, 0] == s and a[1, 1] == c, (t, a[1], c, s)


def pin_identity_and_scaling(o):
    """theta = 0 with s = 1 is the identity bit for bit; theta = 0 alone is x / s and W * s."""
    rng = _rng(1)
    D, K = 256, 3
    pairs, _, scale = _random_transform(rng, D, K)
    theta0 = np.zeros((K, D // 2), np.float32)
    x = rng.normal(0, 1, (3, D)).astype(np.float16).astype(np.float64)
    W = rng.normal(0, 0.02, (5, D)).astype(np.float16).astype(np.float64)
    ones = np.ones(D, np.float32)
    assert np.array_equal(o.transform_activations(x, pairs, theta0, ones), x)
    assert np.array_equal(o.fold_weights(W, pairs, theta0, ones), W)
    assert np.array_equal(o.transform_activations(x, pairs, theta0, scale), x / scale.astype(np.float64))
    assert np.array_equal(o.fold_weights(W, pairs, theta0, scale), W * scale.astype(np.float64))


def pin_pair_norms(o):
    """Each stage keeps every pair's norm, up to the float32 rounding of (cos, sin)."""
    rng = _rng(2)
    D = 128
    pairs, theta, _ = _random_transform(rng, D, 1)
    ones = np.ones(D, np.float32)
    x = rng.normal(0, 1, (4, D))
    a = o.transform_activations(x, pairs, theta, ones)
    i, j = pairs[0, :, 0], pairs[0, :, 1]
    t = theta[0].astype(np.float64)
    c = np.cos(t).astype(np.float32).astype(np.float64)
    s = np.sin(t).astype(np.float32).astype(np.float64)
    assert np.all(np.abs(c * c + s * s - 1.0) <= 2.0 ** -23)
    before = np.hypot(x[:, i], x[:, j])
    after = np.hypot(a[:, i], a[:, j])
    assert np.allclose(after, before * np.sqrt(c * c + s * s), rtol=1e-14, atol=0), np.abs(after / before - 1).max()
    assert np.allclose(after, before, rtol=1e-6, atol=0)


def pin_golden_givens(o):
    with open(os.path.join(GOLDEN, "givens_hand_examples.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        pairs = np.array(case["pairs"], np.int32)
        theta = np.array(case["theta"], np.float32)
        scale = np.array(case["scale"], np.float32)
        a = o.transform_activations(np.array(case["x"], np.float64), pairs, theta, scale)
        exp = np.array(case["expected"], np.float64)
        assert np.allclose(a, exp, atol=g["tolerance"], rtol=0), (case["name"], a, exp)


def _dense_stage(D, pairs_k, c_k, s_k):
    G = np.zeros((D, D))
    done = set()
    for (i, j), c, s in zip(pairs_k, c_k, s_k):
        G[i, i] = c
        G[i, j] = s
        G[j, i] = -s
        G[j, j] = c
        done.update((int(i), int(j)))
    assert len(done) == D
    return G


def pin_dense_bruteforce(o):
    """D = 8: the stages equal T_act = diag(1/s) G_K ... G_1 built as dense matrices, and
    the weight side equals T_w = diag(s) G_K ... G_1, with T_act^T T_w ~ I."""
    rng = _rng(3)
    D, K = 8, 4
    pairs, theta, scale = _random_transform(rng, D, K)
    c = np.array([[float(np.float32(math.cos(float(t)))) for t in row] for row in theta])
    s = np.array([[float(np.float32(math.sin(float(t)))) for t in row] for row in theta])
    G = np.eye(D)
    for k in range(K):
        G = _dense_stage(D, pairs[k], c[k], s[k]) @ G
    T_act = np.diag(1.0 / scale.astype(np.float64)) @ G
    T_w = np.diag(scale.astype(np.float64)) @ G
    x = rng.normal(0, 1, (5, D))
    W = rng.normal(0, 0.02, (3, D))
    assert np.allclose(o.transform_activations(x, pairs, theta, scale), x @ T_act.T, rtol=1e-12, atol=1e-12)
    assert np.allclose(o.fold_weights(W, pairs, theta, scale), W @ T_w.T, rtol=1e-12, atol=1e-14)
    assert np.allclose(T_act.T @ T_w, np.eye(D), atol=1e-6)


def pin_sequential_pairs(o):
    """Disjoint pairs: updating them one at a time (pure Python) gives the same bits."""
    rng = _rng(4)
    D, K = 16, 3
    pairs, theta, scale = _random_transform(rng, D, K)
    x = rng.normal(0, 1, D)
    v = [float(t) for t in x]
    for k in range(K):
        for (i, j), t in zip(pairs[k], theta[k]):
            c = float(np.float32(math.cos(float(t))))
            s = float(np.float32(math.sin(float(t))))
            vi, vj = v[i], v[j]
            v[i] = c * vi + s * vj
            v[j] = c * vj - s * vi
    v = [vv / float(sc) for vv, sc in zip(v, scale)]
    a = o.transform_activations(x[None, :], pairs, theta, scale)[0]
    assert np.array_equal(a, np.array(v)), np.abs(a - v).max()


def pin_invariance(o):
    """The unquantized folded weights reproduce x.W^T to 1e-6 relative."""
    rng = _rng(5)
    for D, K, N in ((256, 2, 64), (1536, 8, 32)):
        pairs, theta, scale = _random_transform(rng, D, K)
        x = rng.normal(0, 1, (4, D))
        x[:, rng.choice(D, 5, replace=False)] *= 30
        W = rng.normal(0, 0.02, (N, D))
        ref = x @ W.T
        got = o.transform_activations(x, pairs, theta, scale) @ o.fold_weights(W, pairs, theta, scale).T
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel <= 1e-6, rel
        assert np.abs(got - ref).max() <= 1e-6 * np.abs(ref).max() * 4


def pin_forward_inverse(o):
    rng = _rng(6)
    D, K = 512, 8
    pairs, theta, scale = _random_transform(rng, D, K)
    x = rng.normal(0, 1, (3, D))
    back = o.untransform_activations(o.transform_activations(x, pairs, theta, scale), pairs, theta, scale)
    assert np.linalg.norm(back - x) / np.linalg.norm(x) <= 1e-6
    assert np.abs(back - x).max() <= 1e-6 * np.abs(x).max()


def pin_matching_check(o):
    D = 8
    good = np.array([[[0, 1], [2, 3], [4, 5], [6, 7]]], np.int32)
    o.check_stage_pairs(good, D)
    bad = [
        np.array([[[0, 1], [1, 3], [4, 5], [6, 7]]], np.int32),  # channel 1 twice, 2 missing
        np.array([[[0, 1], [2, 3], [4, 5], [6, 8]]], np.int32),  # out of range
        np.array([[[0, 1], [2, 3], [4, 5]]], np.int32),  # too few pairs
    ]
    for b in bad:
        try:
            o.check_stage_pairs(b, D)
        except ValueError:
            continue
        raise AssertionError(f"accepted a non-matching stage {b.tolist()}")


# ----------------------------------------------------------------------------- #
# Quantizer, packing, dequantization, linears
# ----------------------------------------------------------------------------- #

def pin_quantizer_closed_form(o):
    """b_k = (k mod 16 - z0) * delta, delta a power of two: codes k mod 16, zero z0,
    scale delta, exact dequantization."""
    rows = []
    expect_z, expect_d = [], []
    for z0, e in ((0, -7), (5, -9), (15, -4), (8, -12)):
        d = 2.0 ** e
        k = np.arange(128)
        rows.append(((k % 16) - z0) * d)
        expect_z.append(z0)
        expect_d.append(d)
    b = np.array(rows)
    q, sc, z = o.quantize_groups(b)
    assert np.array_equal(q, np.tile(np.arange(128) % 16, (4, 1)).astype(np.uint8)), q[:, :20]
    assert np.array_equal(z[:, 0].astype(np.float64), np.array(expect_z, np.float64))
    assert np.array_equal(sc[:, 0].astype(np.float64), np.array(expect_d))
    deq = o.dequantize(o.pack_nibbles(q), sc, z)
    assert np.array_equal(deq, b)


def pin_quantizer_golden(o):
    with open(os.path.join(GOLDEN, "quantizer_hand_examples.json")) as f:
        g = json.load(f)
    b = np.full((1, 128), g["fill"])
    for k, v in g["group_values"].items():
        b[0, int(k)] = v
    q, sc, z = o.quantize_groups(b)
    assert float(sc[0, 0]) == g["expected_scale"], float(sc[0, 0])
    assert float(z[0, 0]) == g["expected_zero"], float(z[0, 0])
    for k, v in g["expected_codes"].items():
        assert int(q[0, int(k)]) == v, (k, int(q[0, int(k)]), v)


def pin_quantizer_ties_and_bound(o):
    """Half-way codes round to even; the min/max quantizer's error is at most about
    half a step when the group straddles zero; a constant group takes the 1e-5 floor."""
    d = 2.0 ** -6
    b = np.zeros((1, 128))
    b[0, 0], b[0, 1] = -8 * d, 7 * d  # range 15 d -> scale d, z = 8
    b[0, 2], b[0, 3], b[0, 4], b[0, 5] = 0.5 * d, 1.5 * d, 2.5 * d, -0.5 * d
    q, sc, z = o.quantize_groups(b)
    assert float(sc[0, 0]) == d and float(z[0, 0]) == 8
    assert [int(v) for v in q[0, 2:6]] == [8, 10, 10, 8], q[0, :6]
    rng = _rng(7)
    w = rng.normal(0, 0.02, (64, 512))
    w[:, ::37] *= 10
    q, sc, z = o.quantize_groups(w)
    deq = o.dequantize(o.pack_nibbles(q), sc, z)
    step = np.repeat(sc.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(deq - w) <= 0.5075 * step), (np.abs(deq - w) / step).max()
    const = np.zeros((2, 128))
    const[1] = 3 * float(np.float16(1e-5))
    q, sc, z = o.quantize_groups(const)
    assert float(sc[0, 0]) == float(np.float16(1e-5)) and float(z[0, 0]) == 0
    assert np.all(q[0] == 0) and np.all(q[1] == 3)


def pin_pack_layout(o):
    q = np.array([[1, 2, 3, 4, 15, 0, 0, 15]], np.uint8)
    packed = o.pack_nibbles(q)
    assert packed.tolist() == [[0x21, 0x43, 0x0F, 0xF0]], [hex(v) for v in packed[0]]
    rng = _rng(8)
    qq = rng.integers(0, 16, (3, 256)).astype(np.uint8)
    assert np.array_equal(o.unpack_nibbles(o.pack_nibbles(qq)), qq)


def pin_linear_bruteforce(o):
    """y = x.deq^T against a pure-Python triple loop; K = 0 with s = 1 makes the rotated
    linear the plain one, bit for bit."""
    rng = _rng(9)
    M, D, N = 2, 128, 3
    x = rng.normal(0, 1, (M, D)).astype(np.float16).astype(np.float64)
    q = rng.integers(0, 16, (N, D)).astype(np.uint8)
    sc = np.array([[0.01], [0.02], [0.005]], np.float16)
    z = np.array([[3], [8], [12]], np.float16)
    qw = o.pack_nibbles(q)
    y = o.w4a16_linear(x, qw, sc, z)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for d in range(D):
                acc += float(x[m, d]) * ((int(q[n, d]) - float(z[n, 0])) * float(sc[n, 0]))
            assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc)), (m, n, y[m, n], acc)
    pairs = np.zeros((0, D // 2, 2), np.int32)
    theta = np.zeros((0, D // 2), np.float32)
    ones = np.ones(D, np.float32)
    assert np.array_equal(o.rotated_linear(x, pairs, theta, ones, qw, sc, z), y)


def pin_pack_end_to_end(o):
    """Packing the folded weights then dequantizing stays within the quantizer's bound of
    the exactly folded weights, and the rotated linear then tracks x.W^T."""
    rng = _rng(10)
    D, K, N, M = 384, 4, 40, 3
    pairs, theta, scale = _random_transform(rng, D, K)
    W = rng.normal(0, 0.02, (N, D)).astype(np.float16)
    x = rng.normal(0, 1, (M, D)).astype(np.float16)
    qw, sc, z = o.pack_weights(W, pairs, theta, scale)
    b = o.fold_weights(W, pairs, theta, scale)
    deq = o.dequantize(qw, sc, z)
    step = np.repeat(sc.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(deq - b) <= 0.5075 * step)
    y = o.rotated_linear(x, pairs, theta, scale, qw, sc, z)
    a = o.transform_activations(x, pairs, theta, scale)
    assert np.allclose(y, a @ deq.T, rtol=1e-12, atol=1e-12)
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 0.2  # INT4 noise, not a wrong transform


ALL_PINS = [
    pin_f16_rounding, pin_givens_closed_form, pin_identity_and_scaling, pin_pair_norms,
    pin_golden_givens, pin_dense_bruteforce, pin_sequential_pairs, pin_invariance,
    pin_forward_inverse, pin_matching_check, pin_quantizer_closed_form, pin_quantizer_golden,
    pin_quantizer_ties_and_bound, pin_pack_layout, pin_linear_bruteforce, pin_pack_end_to_end,
]
