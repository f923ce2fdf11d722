"""GPU parity on the quantizer's edge cases: crafted weight groups that reach every branch of the
min/max INT4 quantizer, run through pack (bit-exact against the oracle), the decode-shaped linear
(M = 1, 4, 16) and the GEMM (M = 64 and 300, split and unsplit reductions).

The quantizer is the one the pages' INT4 group-128 weights go through ("ParoQuant: pairwise
rotations that survive deployment", section "My reduced-calibration experiment": INT4, group
size 128; section "A rotation small enough to execute": the transformed weights are folded and
quantized at build time). The group kinds below make it:
  * clip the zero-point at 0 (all-positive groups) and at 15 (all-negative groups), and clip
    codes at 15 and at 0 (the far ends of those groups);
  * hit the 1e-5 scale floor (constant groups, all-zero groups and rows, groups whose range is
    below 15e-5), whose float16 scale is subnormal;
  * round exact halves, of codes and of the zero-point, to even;
  * put an outlier group (scale near 1) next to a floor group (scale 1e-5), so the GEMM's
    per-group rescale of its accumulators runs at ratios of about 1e5 both ways.
To control the folded weights exactly, the transforms here are exact: no stages (K = 0), or
stages whose angles are all 0 (cos = 1, sin = 0), and channel scales that are powers of two.
A third set uses a random transform with all-zero rows (a zero row stays zero).
"""
import dataclasses

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
rl = pytest.importorskip("rotated_linear_amd")

D = 1024  # eight 128-channel groups per row
N = 200
DELTA = 2.0 ** -6  # float16-exact step of the tie groups


def _group(kind, rng):
    """128 float16-representable values of one crafted group."""
    if kind == 0:  # ordinary: straddles zero
        v = rng.normal(0.0, 0.02, 128)
    elif kind == 1:  # all positive: z clips to 0, the top codes clip to 15
        v = rng.uniform(0.01, 0.5, 128)
    elif kind == 2:  # all negative: z clips to 15, the bottom codes clip to 0
        v = rng.uniform(-0.5, -0.01, 128)
    elif kind == 3:  # constant: scale floor, z and every code clipped
        v = np.full(128, rng.choice([-0.3, 0.3, 1.5]))
    elif kind == 4:  # all zero: scale floor, z = 0, codes 0
        v = np.zeros(128)
    elif kind == 5:  # exact halves: lo = 0, hi = 15 DELTA -> scale DELTA, b / scale = k + 1/2
        v = (rng.integers(0, 15, 128) + 0.5) * DELTA
        v[:2] = (0.0, 15 * DELTA)
    elif kind == 6:  # exact halves around zero: lo = -7.5 DELTA (z = rint(7.5) = 8), hi = 7.5 DELTA
        v = (rng.integers(-8, 8, 128) + 0.5) * DELTA
        v[:2] = (-7.5 * DELTA, 7.5 * DELTA)
    elif kind == 7:  # outlier: scale about 1
        v = rng.normal(0.0, 3.0, 128)
    else:  # tiny range (below 15e-5): the scale floor with codes spread out
        v = rng.normal(0.0, 1.5e-5, 128)
    return v.astype(np.float16)


def crafted_weights(seed):
    """W float16 [N][D]: row n, group g of kind (n + 3 g) % 9; rows 5 and 77 all zero; rows
    9 and 10 alternate outlier and floor groups (both orders)."""
    rng = np.random.default_rng(seed)
    Wm = np.zeros((N, D), np.float16)
    for n in range(N):
        for g in range(D // 128):
            kind = (n + 3 * g) % 9
            if n in (9, 10):
                kind = (7, 3, 7, 4, 7, 8, 4, 7)[g] if n == 9 else (3, 7, 8, 7, 4, 7, 3, 7)[g]
            Wm[n, g * 128:(g + 1) * 128] = _group(kind, rng)
    Wm[5] = 0
    Wm[77] = 0
    return Wm


def _inputs(kind, M=300):
    """Activations x (N(0,1), float16) and a transform of the named kind with crafted weights."""
    base = W.custom_linear(900 + kind, M, D, N, 8)
    rng = np.random.default_rng(1000 + kind)
    Wm = crafted_weights(kind)
    if kind == 0:  # no stages, s = 1: the folded weights are W itself (exact halves stay halves)
        pairs, theta, scale = base.pairs[:0], base.theta[:0], np.ones(D, np.float32)
    elif kind == 1:  # three stages of zero angles (the identity) and power-of-two scales
        pairs = base.pairs[:3]
        theta = np.zeros_like(base.theta[:3])
        scale = rng.choice([0.5, 1.0, 2.0], D).astype(np.float32)
    else:  # a random transform; only the zero rows stay crafted
        pairs, theta, scale = base.pairs, base.theta, base.scale
    spec = dataclasses.replace(base.spec, K=pairs.shape[0])
    return dataclasses.replace(base, spec=spec, W=Wm, pairs=pairs, theta=theta, scale=scale)


def _coverage(L, q, sc, z):
    """The branches the crafted groups reach in the oracle's quantizer (so a change to the
    recipe that stops reaching one fails here, not silently)."""
    b = O.fold_weights(L.W, L.pairs, L.theta, L.scale).reshape(N, D // 128, 128)
    lo, hi = b.min(axis=2), b.max(axis=2)
    floor = sc.astype(np.float64) == np.float64(np.float16(1e-5))
    raw_z = np.rint(-lo / sc.astype(np.float64))
    raw_q = np.rint(b / sc.astype(np.float64)[:, :, None]) + z.astype(np.float64)[:, :, None]
    return {"z clipped to 0": bool((raw_z < 0).any()), "z clipped to 15": bool((raw_z > 15).any()),
            "q clipped to 15": bool((raw_q > 15).any()), "q clipped to 0": bool((raw_q < 0).any()),
            "scale floor": bool(floor.any()), "floor next to outlier": bool((floor[:, :-1] & (sc[:, 1:] > 0.5)).any()
                                                                          and (floor[:, 1:] & (sc[:, :-1] > 0.5)).any()),
            "subnormal scale": bool((np.abs(sc.astype(np.float64)) < 2.0 ** -14).any()),
            "code ties": bool((np.abs(b / sc.astype(np.float64)[:, :, None] % 1.0 - 0.5) == 0).any()),
            "zero ties": bool((np.abs((-lo / sc.astype(np.float64)) % 1.0 - 0.5) == 0).any())}


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_crafted_pack_bitexact(kind):
    L = _inputs(kind)
    C.log(f"crafted pack kind={kind} K={L.spec.K} D={D} N={N}")
    rot = rl.paro_rotation_prepare(L.pairs, L.theta, L.scale)
    qw, sc, z = C.host_weights(rl.paro_pack_weights(rot, C.dev(L.W, torch)))
    oq, osc, oz = O.pack_weights(L.W, L.pairs, L.theta, L.scale)
    assert np.array_equal(qw, oq), f"qweight differs in {(qw != oq).sum()} bytes"
    assert np.array_equal(sc.view(np.uint16), osc.view(np.uint16)), "scales differ"
    assert np.array_equal(z.astype(np.float64), oz.astype(np.float64)), "zeros differ"
    cov = _coverage(L, O.unpack_nibbles(oq), osc, oz)
    if kind == 0:  # every branch, ties included
        assert all(cov.values()), cov
    elif kind == 1:
        assert all(v for k, v in cov.items() if "ties" not in k), cov
    else:
        assert cov["scale floor"], cov


def _linear_bar(y, ref, what):
    mx, rel = C.linear_metrics(y, ref)
    assert mx <= C.MAX_ABS and rel <= C.REL_L2, f"{what}: max-abs {mx:.3e} rel-L2 {rel:.3e}"


@pytest.mark.parametrize("kind", [0, 1, 2])
@pytest.mark.parametrize("M", [1, 4, 16, 64, 300])
def test_crafted_linears(kind, M):
    """Both linears on crafted weights, against the oracle: the decode kernel (M <= 16) and the
    GEMM (M = 64, 300) with and without its split reduction."""
    L = _inputs(kind)
    C.log(f"crafted linear kind={kind} M={M}")
    rot = rl.paro_rotation_prepare(L.pairs, L.theta, L.scale)
    w = rl.paro_pack_weights(rot, C.dev(L.W, torch))
    oq, osc, oz = O.pack_weights(L.W, L.pairs, L.theta, L.scale)
    assert np.array_equal(C.from_blocked(C.host(w[0])), oq)
    deq = O.dequantize(oq, osc, oz)
    x = L.x[:M]
    xd = C.dev(x, torch)
    a = O.transform_activations(x, L.pairs, L.theta, L.scale)
    ref_rot = O.f16_rne(a).astype(np.float64) @ deq.T
    ref_plain = x.astype(np.float64) @ deq.T
    # With an exact transform (kinds 0 and 1) x' is exactly float16(a). With a random one, the
    # float32 transform lands on the other float16 neighbour for a few elements (the rotate tests
    # bound it), and the crafted weights (|q - z| * scale up to about 20) magnify one float16
    # spacing of x' past 1e-2: there the rotated linear is held to the propagated bound instead,
    # |y - a . deq^T| <= rotate_bound(a) . |deq|^T + the float32 summation term.
    exact = kind != 2
    bound = None
    if not exact:
        rb = C.rotate_bound(a, x.astype(np.float64), L.scale, L.spec.K)
        bound = rb @ np.abs(deq).T + (128 + D // 128 + 4) * 2.0 ** -24 * (np.abs(a) + rb) @ np.abs(deq).T
        ref_exact = a @ deq.T
    need = rl.paro_workspace_bytes(M, D, N)
    for ws in (None, torch.empty(max(need, 256), dtype=torch.uint8, device="cuda"),
               torch.empty(256, dtype=torch.uint8, device="cuda")):
        tag = "default ws" if ws is None else f"ws {ws.numel()} B"
        _linear_bar(C.host(rl.paro_w4a16_linear(xd, *w, out_dtype=torch.float32, ws=ws)), ref_plain,
                    f"w4a16 ({tag})")
        if ws is None or ws.numel() >= need:
            y = C.host(rl.paro_rotated_linear(rot, xd, *w, out_dtype=torch.float32, ws=ws))
            if exact:
                _linear_bar(y, ref_rot, f"rotated ({tag})")
            else:
                over = C.over_bound(y - ref_exact, bound)
                assert over <= 1.0, f"rotated ({tag}): error {over:.3f}x its propagated bound"
                assert C.linear_metrics(y, ref_rot)[1] <= C.REL_L2


@pytest.mark.parametrize("M", [1, 4, 16, 64, 300])
def test_zero_scales_contribute_nothing(M):
    """A group whose scale is zero contributes nothing (the linear's formula). paro_pack_weights
    never writes one (its floor is fp16(1e-5)), so the packed weights are edited here: every
    fifth group's scale, the first group of row 3 and every group of row 4 set to zero."""
    L = _inputs(0)
    C.log(f"zero scales M={M}")
    oq, osc, oz = O.pack_weights(L.W, L.pairs, L.theta, L.scale)
    osc = osc.copy()
    osc.reshape(-1)[::5] = 0
    osc[3, 0] = 0
    osc[4, :] = 0
    deq = O.dequantize(oq, osc, oz)
    x = L.x[:M]
    xd = C.dev(x, torch)
    w = C.dev_weights((oq, osc, oz), torch)
    ref = x.astype(np.float64) @ deq.T
    need = rl.paro_workspace_bytes(M, D, N)
    for ws in (torch.empty(max(need, 256), dtype=torch.uint8, device="cuda"),
               torch.empty(256, dtype=torch.uint8, device="cuda")):
        y = C.host(rl.paro_w4a16_linear(xd, *w, out_dtype=torch.float32, ws=ws))
        assert np.isfinite(y).all()
        assert np.all(y[:, 4] == 0.0), "a row whose scales are all zero must give exact zeros"
        _linear_bar(y, ref, f"zero scales (ws {ws.numel()} B)")
