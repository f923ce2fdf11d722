"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars:
  * pack: qweight bytes, scales and zeros bit-identical to the oracle;
  * rotate: every element within ``rotate_bound`` of the float64 transform, and few
    elements off the float16 rounding of the float64 transform (``C.rotate_off_cap``: an
    emulation of the kernel's float32 sequence puts 0.06% of elements off at K = 8, growing
    about linearly with K);
  * linears (spec bar): max-abs <= 1e-2 and relative L2 <= 2e-3, with the
    float32-output epilogue, against the oracle applied to the same dequantized
    weights and -- for the rotated linear -- the same float16 activations the
    GEMM consumes (f16_rne of the float64 transform); the production float16
    output is also held to relative L2 <= 2e-3 against the unrounded float64 path and, element
    by element, to ``C.fp16_path_bound`` (the exact effect of rounding x' to float16, float32
    summation, the output's rounding); on the configured workloads also to max-abs <= 1e-2 on
    the outputs with |y| < 16 (above, one float16 spacing exceeds 1e-2).
Full-size workloads are checked on sampled weight rows / token rows, always
including the first and last (ragged) ones.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
rl = pytest.importorskip("rotated_linear_amd")


def _rot(L):
    return rl.paro_rotation_prepare(L.pairs, L.theta, L.scale)


# --------------------------------------------------------------------------- #
# pack: bit-exact
# --------------------------------------------------------------------------- #

PACK_CASES = [(1, 0), (2, 0), (2, 1), (3, 0), (4, 0)] + [(5, i) for i in range(7)]


@pytest.mark.parametrize("wid,index", PACK_CASES)
def test_pack_bitexact(wid, index):
    L = C.linear_inputs(wid, index)
    C.log(f"pack wid={wid} linear={L.spec.name} N={L.spec.N} D={L.spec.D} K={L.spec.K}")
    rot = _rot(L)
    qw, sc, z = rl.paro_pack_weights(rot, C.dev(L.W, torch))
    torch.cuda.synchronize()
    rows = C.sample_rows(L.spec.N, 384, seed=wid * 10 + index)
    key = None if len(rows) == L.spec.N else tuple(int(r) for r in rows)
    oq, osc, oz = C.oracle_pack_rows(wid, index, key)
    gq, gsc, gz = (t[rows] for t in C.host_weights((qw, sc, z)))
    assert np.array_equal(gq, oq), f"qweight differs in {(gq != oq).sum()} bytes"
    assert np.array_equal(gsc.view(np.uint16), osc.view(np.uint16)), "scales differ"
    assert np.array_equal(gz.astype(np.float64), oz.astype(np.float64)), "zeros differ"


def test_pack_pair_order_and_roles_do_not_matter():
    """Disjoint pairs: reordering the pairs of a stage, or swapping (i, j) with theta -> -theta,
    leaves the folded weights bit-identical (section "A rotation small enough to execute")."""
    L = W.custom_linear(31, 1, 512, 96, 4)
    C.log("pack pair order / role swap D=512 N=96 K=4")
    rng = np.random.default_rng(5)
    pairs2, theta2 = L.pairs.copy(), L.theta.copy()
    for k in range(L.pairs.shape[0]):
        perm = rng.permutation(L.pairs.shape[1])
        pairs2[k], theta2[k] = pairs2[k][perm], theta2[k][perm]
        flip = rng.random(L.pairs.shape[1]) < 0.5
        pairs2[k][flip] = pairs2[k][flip][:, ::-1]
        theta2[k][flip] = -theta2[k][flip]
    Wd = C.dev(L.W, torch)
    a = [C.host(t) for t in rl.paro_pack_weights(_rot(L), Wd)]
    b = [C.host(t) for t in rl.paro_pack_weights(rl.paro_rotation_prepare(pairs2, theta2, L.scale), Wd)]
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_pack_edge_shapes():
    for (M, D, N, K) in ((1, 128, 1, 0), (1, 128, 3, 1), (1, 16384, 2, 2), (1, 640, 33, 8)):
        L = W.custom_linear(7, M, D, N, K)
        C.log(f"pack edge D={D} N={N} K={K}")
        qw, sc, z = rl.paro_pack_weights(_rot(L), C.dev(L.W, torch))
        oq, osc, oz = O.pack_weights(L.W, L.pairs, L.theta, L.scale)
        assert np.array_equal(C.from_blocked(C.host(qw)), oq)
        assert np.array_equal(C.host(qw), C.to_blocked(oq))
        assert np.array_equal(C.host(sc).view(np.uint16), osc.view(np.uint16))
        assert np.array_equal(C.host(z).astype(np.float64), oz.astype(np.float64))


# --------------------------------------------------------------------------- #
# rotate
# --------------------------------------------------------------------------- #

def _check_rotate(L, x):
    rot = _rot(L)
    got = C.host(rl.paro_rotate(rot, C.dev(x, torch))).astype(np.float64)
    a = O.transform_activations(x, L.pairs, L.theta, L.scale)
    bound = C.rotate_bound(a, x.astype(np.float64), L.scale, L.spec.K)
    err = np.abs(got - a)
    worst = float((err / bound).max())
    assert worst <= 1.0, f"rotate error {worst:.3f}x the bound"
    _check_off_rate(got, a, L.spec.K)
    return got


def _check_off_rate(got, a, K):
    off = int((got != O.f16_rne(a).astype(np.float64)).sum())
    cap = C.rotate_off_cap(a.size, K)
    C.log(f"  rotate: {off} of {a.size} elements ({off / a.size:.4%}) off fp16(float64 transform), cap {cap}")
    assert off <= cap, f"{off} of {a.size} elements off the float16 rounding of the float64 transform (cap {cap})"


ROT_CASES = [(1, 0, 4), (2, 0, 1), (2, 1, 4), (2, 3, 16), (3, 0, 1), (3, 0, 16), (3, 0, 256), (4, 0, 2048),
             (5, 0, 64), (5, 6, 64), (5, 4, 4096)]


@pytest.mark.parametrize("wid,index,M", ROT_CASES)
def test_rotate_parity(wid, index, M):
    L = C.linear_inputs(wid, index)
    C.log(f"rotate wid={wid} linear={L.spec.name} M={M} D={L.spec.D} K={L.spec.K}")
    x = L.x[:M]
    if M > 512:  # full-size batch: compare a row sample (rows are independent)
        rot = _rot(L)
        got = C.host(rl.paro_rotate(rot, C.dev(x, torch))).astype(np.float64)
        rows = C.sample_rows(M, 128, seed=M)
        a = O.transform_activations(x[rows], L.pairs, L.theta, L.scale)
        bound = C.rotate_bound(a, x[rows].astype(np.float64), L.scale, L.spec.K)
        assert float((np.abs(got[rows] - a) / bound).max()) <= 1.0
        _check_off_rate(got[rows], a, L.spec.K)
    else:
        _check_rotate(L, x)


def test_rotate_identity_and_order():
    L = W.custom_linear(3, 5, 384, 8, 3)
    C.log("rotate identity / pair-order shuffle D=384 M=5")
    zero = np.zeros_like(L.theta)
    ones = np.ones_like(L.scale)
    xd = C.dev(L.x, torch)
    same = C.host(rl.paro_rotate(rl.paro_rotation_prepare(L.pairs, zero, ones), xd))
    assert np.array_equal(same.view(np.uint16), L.x.view(np.uint16)), "theta=0, s=1 must be the identity"
    base = C.host(rl.paro_rotate(_rot(L), xd))
    rng = np.random.default_rng(9)
    p2, t2 = L.pairs.copy(), L.theta.copy()
    for k in range(L.pairs.shape[0]):
        perm = rng.permutation(L.pairs.shape[1])
        p2[k], t2[k] = p2[k][perm], t2[k][perm]
    shuf = C.host(rl.paro_rotate(rl.paro_rotation_prepare(p2, t2, L.scale), xd))
    assert np.array_equal(base.view(np.uint16), shuf.view(np.uint16)), "pair order within a stage changed bits"
    again = C.host(rl.paro_rotate(_rot(L), xd))
    assert np.array_equal(base.view(np.uint16), again.view(np.uint16)), "not deterministic"


@pytest.mark.parametrize("M,D,K", [(1, 128, 0), (3, 128, 1), (5, 384, 3), (7, 16384, 2), (9, 1280, 8),
                                   (130, 640, 5),
                                   # one wide row per 1024-thread workgroup: exact (14336) and not
                                   (100, 9344, 3), (33, 14336, 2), (40, 12544, 8), (3, 8960, 8), (200, 6272, 4),
                                   # the most stages (rolled stage loop), one past the unrolled count
                                   (20, 1024, 64), (6, 2048, 9),
                                   # rows per block 2 and 4, widths at and past the 4-row limit
                                   (300, 1536, 8), (600, 9216, 3), (1100, 9216, 2), (520, 9344, 2)])
def test_rotate_edge_shapes(M, D, K):
    L = W.custom_linear(11, M, D, 4, K)
    C.log(f"rotate edge M={M} D={D} K={K}")
    _check_rotate(L, L.x)


# --------------------------------------------------------------------------- #
# linears
# --------------------------------------------------------------------------- #

def _linear_case(L, M, rows_w, oracle_pack, gpu_weights, configured=True):
    """Run both linears on the GPU and compare against the oracle on the sampled weight rows."""
    x = L.x[:M]
    xd = C.dev(x, torch)
    rot = _rot(L)
    qw, sc, z = gpu_weights
    y32 = C.host(rl.paro_rotated_linear(rot, xd, qw, sc, z, out_dtype=torch.float32))
    y16 = C.host(rl.paro_rotated_linear(rot, xd, qw, sc, z, out_dtype=torch.float16))
    p32 = C.host(rl.paro_w4a16_linear(xd, qw, sc, z, out_dtype=torch.float32))
    oq, osc, oz = oracle_pack
    a = O.transform_activations(x, L.pairs, L.theta, L.scale)
    deq = O.dequantize(oq, osc, oz)
    ref_fused = O.f16_rne(a).astype(np.float64) @ deq.T
    ref_exact = a @ deq.T
    ref_plain = x.astype(np.float64) @ deq.T
    mx, rel = C.linear_metrics(y32[:, rows_w], ref_fused)
    assert mx <= C.MAX_ABS and rel <= C.REL_L2, f"rotated linear (fp32 out): max-abs {mx:.3e} rel-L2 {rel:.3e}"
    mx2, rel2 = C.linear_metrics(y16[:, rows_w], ref_exact)
    assert rel2 <= C.REL_L2, f"rotated linear (fp16 out vs float64 path): rel-L2 {rel2:.3e} (max-abs {mx2:.3e})"
    over = C.over_bound(y16[:, rows_w] - ref_exact, C.fp16_path_bound(a, deq, ref_exact))
    assert over <= 1.0, f"rotated linear (fp16 out vs float64 path): error {over:.3f}x its bound"
    mx16 = C.masked_max_abs(y16[:, rows_w], ref_exact, 16.0)
    if configured:  # the workloads' bar; at other shapes (D up to 16384) the bound above holds
        assert mx16 <= C.MAX_ABS, f"rotated linear (fp16 out vs float64 path): max-abs {mx16:.3e} where |y| < 16"
    mx3, rel3 = C.linear_metrics(p32[:, rows_w], ref_plain)
    assert mx3 <= C.MAX_ABS and rel3 <= C.REL_L2, f"w4a16 linear: max-abs {mx3:.3e} rel-L2 {rel3:.3e}"
    return mx, rel, mx2, rel2


LIN_CASES = [(1, 0, 4), (2, 0, 1), (2, 0, 4), (2, 0, 16), (2, 1, 1), (2, 1, 16), (2, 3, 4), (3, 0, 1), (3, 0, 16),
             (3, 0, 256), (4, 0, 2048), (5, 0, 64), (5, 1, 64), (5, 4, 64), (5, 6, 64), (5, 3, 4096), (5, 6, 4096)]


@pytest.mark.parametrize("wid,index,M", LIN_CASES)
def test_linear_parity(wid, index, M):
    L = C.linear_inputs(wid, index)
    C.log(f"linear wid={wid} linear={L.spec.name} M={M} N={L.spec.N} D={L.spec.D}")
    N = L.spec.N
    rows_w = C.sample_rows(N, 256, seed=wid * 100 + index)
    key = None if len(rows_w) == N else tuple(int(r) for r in rows_w)
    oracle_pack = C.oracle_pack_rows(wid, index, key)
    if key is None:
        gpu_w = C.dev_weights(oracle_pack, torch)  # the oracle's own packed weights
    else:
        gpu_w = rl.paro_pack_weights(_rot(L), C.dev(L.W, torch))  # full weights; sampled rows checked bit-exact
        assert np.array_equal(C.from_blocked(C.host(gpu_w[0]))[rows_w], oracle_pack[0])
    if M > 512:  # token-row sample for the large prefill batches
        Lm = L
        x_rows = C.sample_rows(M, 96, seed=M + index)
        x = L.x[:M]
        xd = C.dev(x, torch)
        rot = _rot(L)
        y32 = C.host(rl.paro_rotated_linear(rot, xd, *gpu_w, out_dtype=torch.float32))[x_rows][:, rows_w]
        y16 = C.host(rl.paro_rotated_linear(rot, xd, *gpu_w, out_dtype=torch.float16))[x_rows][:, rows_w]
        p32 = C.host(rl.paro_w4a16_linear(xd, *gpu_w, out_dtype=torch.float32))[x_rows][:, rows_w]
        a = O.transform_activations(x[x_rows], Lm.pairs, Lm.theta, Lm.scale)
        deq = O.dequantize(*oracle_pack)
        mx, rel = C.linear_metrics(y32, O.f16_rne(a).astype(np.float64) @ deq.T)
        assert mx <= C.MAX_ABS and rel <= C.REL_L2, f"rotated linear: max-abs {mx:.3e} rel-L2 {rel:.3e}"
        ref_exact = a @ deq.T
        mx2, rel2 = C.linear_metrics(y16, ref_exact)
        mx16 = C.masked_max_abs(y16, ref_exact, 16.0)
        assert rel2 <= C.REL_L2 and mx16 <= C.MAX_ABS, f"fp16 out: rel-L2 {rel2:.3e}, max-abs {mx16:.3e} where |y| < 16"
        assert C.over_bound(y16 - ref_exact, C.fp16_path_bound(a, deq, ref_exact)) <= 1.0
        mx3, rel3 = C.linear_metrics(p32, x[x_rows].astype(np.float64) @ deq.T)
        assert mx3 <= C.MAX_ABS and rel3 <= C.REL_L2, f"w4a16 linear: max-abs {mx3:.3e} rel-L2 {rel3:.3e}"
        C.log(f"  max-abs {mx:.2e} rel-L2 {rel:.2e}")
    else:
        mx, rel, _, _ = _linear_case(L, M, rows_w, oracle_pack, gpu_w)
        C.log(f"  max-abs {mx:.2e} rel-L2 {rel:.2e}")


@pytest.mark.parametrize("M,D,N,K", [(1, 128, 1, 1), (2, 384, 200, 3), (3, 640, 77, 2), (4, 256, 513, 0),
                                     (5, 384, 200, 3), (17, 1280, 130, 4), (33, 512, 64, 2), (65, 768, 96, 8),
                                     (130, 1024, 300, 5), (257, 384, 129, 1), (1, 16384, 40, 2), (6, 16384, 20, 2),
                                     # a few dozen rows: one group, ragged columns, deep reductions
                                     (20, 128, 1, 2), (40, 1152, 513, 0), (48, 16384, 300, 1), (64, 4096, 257, 3),
                                     (50, 2304, 1000, 8),
                                     # deep transforms on the two-kernel path
                                     (3, 512, 100, 64), (40, 1024, 200, 33)])
def test_linear_edge_shapes(M, D, N, K):
    L = W.custom_linear(21, M, D, N, K)
    C.log(f"linear edge M={M} D={D} N={N} K={K}")
    op = O.pack_weights(L.W, L.pairs, L.theta, L.scale)
    _linear_case(L, M, np.arange(N), op, C.dev_weights(op, torch), configured=False)


@pytest.mark.parametrize("M", [1, 3, 4, 16, 200])
def test_identity_transform_matches_plain_linear(M):
    """K = 0 with s = 1: the rotated linear must equal the plain INT4 linear bit for bit."""
    L = W.custom_linear(41, M, 1536, 300, 0)
    C.log(f"identity transform M={M}")
    rot = rl.paro_rotation_prepare(L.pairs, L.theta, np.ones_like(L.scale))
    qw, sc, z = rl.paro_pack_weights(rot, C.dev(L.W, torch))
    xd = C.dev(L.x, torch)
    for dt in (torch.float16, torch.float32):
        a = C.host(rl.paro_rotated_linear(rot, xd, qw, sc, z, out_dtype=dt))
        b = C.host(rl.paro_w4a16_linear(xd, qw, sc, z, out_dtype=dt))
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_inside_and_separate_transform_agree():
    """A call whose later 4-row units would re-read too many weights runs its transform as its
    own launch (M = 16, 10 MB of weights here); a 4-row call on the same weights runs it inside
    the decode kernel. Both paths round x' once to float16 and sum in the same order, so the
    first 4 rows agree bit for bit; the 16-row call also meets the oracle bar."""
    L = W.custom_linear(43, 16, 1536, 12000, 8)
    C.log("transform inside vs separate launch, D=1536 N=12000")
    rot = _rot(L)
    qw, sc, z = rl.paro_pack_weights(rot, C.dev(L.W, torch))
    xd = C.dev(L.x, torch)
    for dt in (torch.float16, torch.float32):
        a = C.host(rl.paro_rotated_linear(rot, xd, qw, sc, z, out_dtype=dt))
        b = C.host(rl.paro_rotated_linear(rot, xd[:4].contiguous(), qw, sc, z, out_dtype=dt))
        assert np.array_equal(a[:4].view(np.uint8), b.view(np.uint8))
    deq = O.dequantize(*C.host_weights((qw, sc, z)))
    ref = O.f16_rne(O.transform_activations(L.x, L.pairs, L.theta, L.scale)).astype(np.float64) @ deq.T
    mx, rel = C.linear_metrics(a, ref)
    assert mx <= C.MAX_ABS and rel <= C.REL_L2, (mx, rel)


@pytest.mark.parametrize("D,N,K", [(4224, 300, 8), (5120, 2000, 0), (8960, 1536, 8), (9216, 77, 3)])
def test_wide_transform_inside_matches_separate(D, N, K):
    """Rows wider than 4096 channels: a single-row call runs its transform inside the decode
    kernel (one-row units, up to 9 channel pairs per thread per stage), a two-row call as its own
    launch before the linear. Both round x' once to float16 and sum in the same order, so the
    first row agrees bit for bit; the single-row call also meets the oracle bar."""
    L = W.custom_linear(47, 2, D, N, K)
    C.log(f"wide transform inside vs separate launch, D={D} N={N} K={K}")
    rot = _rot(L)
    qw, sc, z = rl.paro_pack_weights(rot, C.dev(L.W, torch))
    xd = C.dev(L.x, torch)
    for dt in (torch.float16, torch.float32):
        a = C.host(rl.paro_rotated_linear(rot, xd[:1].contiguous(), qw, sc, z, out_dtype=dt))
        b = C.host(rl.paro_rotated_linear(rot, xd, qw, sc, z, out_dtype=dt))
        assert np.array_equal(a.view(np.uint8), b[:1].view(np.uint8)), dt
    deq = O.dequantize(*C.host_weights((qw, sc, z)))
    ref = O.f16_rne(O.transform_activations(L.x[:1], L.pairs, L.theta, L.scale)).astype(np.float64) @ deq.T
    mx, rel = C.linear_metrics(a, ref)
    assert mx <= C.MAX_ABS and rel <= C.REL_L2, (mx, rel)


def _wide_sweep(n):
    rng = np.random.default_rng(2024)
    return [(int(128 * rng.integers(33, 73)), int(rng.integers(1, 700)), int(rng.integers(0, 9))) for _ in range(n)]


@pytest.mark.parametrize("D,N,K", _wide_sweep(8))
def test_wide_transform_inside_sweep(D, N, K):
    """Seeded random single-row shapes past 4096 channels (D up to 9216, ragged N, K = 0..8): the
    transform inside the decode kernel agrees bit for bit with the two-launch path of a two-row
    call, and meets the oracle bar."""
    test_wide_transform_inside_matches_separate(D, N, K)


def test_split_reduction_and_fallback():
    """M = 64: with a workspace the reduction over D is split and the float32 partial sums are
    added in split order; without one the call does not split. Both match the oracle, the
    split call is deterministic, and the two differ only in float32 summation order."""
    L = W.custom_linear(43, 64, 4096, 600, 2)
    C.log("split / unsplit reduction M=64 D=4096 N=600")
    op = O.pack_weights(L.W, L.pairs, L.theta, L.scale)
    qw, sc, z = C.dev_weights(op, torch)
    xd = C.dev(L.x, torch)
    need = rl.paro_workspace_bytes(64, 4096, 600)
    ref = L.x.astype(np.float64) @ O.dequantize(*op).T
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    a = C.host(rl.paro_w4a16_linear(xd, qw, sc, z, out_dtype=torch.float32, ws=ws))
    b = C.host(rl.paro_w4a16_linear(xd, qw, sc, z, out_dtype=torch.float32, ws=ws))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    c = C.host(rl.paro_w4a16_linear(xd, qw, sc, z, out_dtype=torch.float32,
                                    ws=torch.empty(256, dtype=torch.uint8, device="cuda")))
    for y in (a, c):
        mx, rel = C.linear_metrics(y, ref)
        assert mx <= C.MAX_ABS and rel <= C.REL_L2, (mx, rel)
    assert np.abs(a - c).max() <= 1e-4 * np.abs(ref).max()


def test_empty_inputs_are_noops():
    L = W.custom_linear(2, 1, 256, 8, 1)
    C.log("empty inputs")
    rot = _rot(L)
    x0 = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    assert rl.paro_rotate(rot, x0).shape == (0, 256)
    qw, sc, z = rl.paro_pack_weights(rot, C.dev(L.W, torch))
    y = torch.full((0, 8), 7.0, dtype=torch.float16, device="cuda")
    rl.paro_rotated_linear(rot, x0, qw, sc, z, out=y)
    sentinel = torch.full((1, 0), 7.0, dtype=torch.float16, device="cuda")
    rl.paro_w4a16_linear(C.dev(L.x, torch), qw[:0], sc[:0], z[:0], out=sentinel)
    torch.cuda.synchronize()


def test_workspace_and_determinism():
    L = C.linear_inputs(4, 0)
    C.log("workspace / determinism down_proj M=300")
    rot = _rot(L)
    qw, sc, z = rl.paro_pack_weights(rot, C.dev(L.W, torch))
    xd = C.dev(L.x[:300], torch)
    need = rl.paro_workspace_bytes(300, L.spec.D, L.spec.N)
    assert need >= 300 * L.spec.D * 2
    with pytest.raises(rl.ParoError):
        rl.paro_rotated_linear(rot, xd, qw, sc, z, ws=torch.empty(need - 256, dtype=torch.uint8, device="cuda"))
    a = C.host(rl.paro_rotated_linear(rot, xd, qw, sc, z))
    b = C.host(rl.paro_rotated_linear(rot, xd, qw, sc, z,
                                      ws=torch.empty(need + 4096, dtype=torch.uint8, device="cuda")))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


# --------------------------------------------------------------------------- #
# batches: one launch for many linears, bit-identical to the single calls
# --------------------------------------------------------------------------- #

def _batch_inputs(specs):
    """specs: (seed, M, D, N, K or None) -> list of (L, rot or None, x, packed weights on the GPU)."""
    out = []
    for seed, M, D, N, K in specs:
        L = W.custom_linear(seed, M, D, N, 0 if K is None else K)
        rot = None if K is None else _rot(L)
        if rot is None:
            qw, sc, z = C.dev_weights(O.pack_weights(L.W, L.pairs[:0], L.theta[:0], np.ones_like(L.scale)), torch)
        else:
            qw, sc, z = rl.paro_pack_weights(rot, C.dev(L.W, torch))
        out.append((L, rot, C.dev(L.x, torch), (qw, sc, z)))
    return out


def _single(rot, xd, w, dt):
    if rot is None:
        return rl.paro_w4a16_linear(xd, *w, out_dtype=dt)
    return rl.paro_rotated_linear(rot, xd, *w, out_dtype=dt)


@pytest.mark.parametrize("specs", [
    # the attention projections of a decode step: q, k, v, o at M = 1, 4, 16 (D = 1536)
    [(60 + i, M, 1536, N, 8) for M in (1, 4, 16) for i, N in enumerate((1536, 256, 256, 1536))],
    # plain and rotated mixed, ragged N, several D, a prefill-sized call and a deep transform
    [(70, 3, 768, 200, 8), (71, 16, 768, 77, None), (72, 5, 2048, 130, 2), (73, 1, 2048, 16, None),
     (74, 40, 768, 96, 8), (75, 2, 768, 64, 12), (76, 7, 8960 // 70 * 70, 33, 8), (77, 1, 4096, 300, 8)],
    # 20 transforms of one D with M > 16 (two batched transform launches of up to 16 jobs),
    # ragged M, K from 0 to 12, plus plain calls in between
    [(90 + i, 17 + 3 * i, 512, 40 + i, [2, 8, 12, 0][i % 4]) for i in range(20)]
    + [(120, 33, 512, 64, None), (121, 300, 512, 96, None), (122, 300, 512, 96, 8)],
    # 40 decode-shaped calls of one D: more units than one decode launch carries (several launches),
    # rotated and plain mixed, M from 1 to 16
    [(200 + i, (1, 2, 4, 16, 3)[i % 5], 512, 24 + 8 * (i % 7), 8 if i % 6 else None) for i in range(40)],
    # decode-shaped calls whose transform runs outside the decode kernel (D > 4096 with more than
    # one row, K > 8): batched transforms, then one decode launch per D over the transformed rows;
    # the single-row calls of D = 4224 run it inside (one-row units)
    [(300 + i, (1, 3, 16, 5)[i % 4], 4224, 40 + 16 * i, 8) for i in range(6)]
    + [(310 + i, (2, 16)[i % 2], 512, 48, 12) for i in range(4)] + [(320, 4, 4224, 64, None)],
    # GEMM-shaped calls of up to 256 rows with different tilings, rotated and plain: grouped
    # launches (one per tiling and x order) and one grouped split reduction
    [(500, 200, 1024, 2048, 8), (501, 20, 1024, 64, 8), (502, 250, 1024, 1536, None), (503, 17, 1024, 4096, None),
     (504, 128, 2048, 256, 4), (505, 64, 4096, 1024, 8), (506, 64, 4096, 1024, None)],
    # long rotated calls (M > 256, prefill-shaped) whose transforms run ahead on the library's
    # second stream while the linears run in order, each waiting for its own transform: 18 of
    # them (more than the 16 ready events, which are then reused), two D, ragged M, plain long
    # calls and short calls in between
    [(600 + i, (257, 300, 513, 384)[i % 4], (512, 1024)[i % 2], 64 + 32 * (i % 3), (8, 2, 12)[i % 3])
     for i in range(18)]
    + [(630, 400, 512, 96, None), (631, 40, 1024, 128, 8), (632, 3, 512, 64, 8), (633, 300, 1024, 64, None)],
    # one layer of the 1.5B-shaped stack at decode M = 1 (q, k, v, o, gate, up, down), as the
    # whole-stack decode step batches it
    [(400 + i, 1, s.D, s.N, s.K) for i, s in enumerate(W.MODEL_LINEARS)],
])
def test_batch_matches_single_calls_bitwise(specs):
    C.log(f"batch of {len(specs)} calls")
    ins = _batch_inputs(specs)
    calls = [(rot, xd, *w) for (L, rot, xd, w) in ins]
    for dt in (torch.float32, torch.float16):
        ys = [C.host(y) for y in rl.paro_linear_batch(calls, out_dtype=dt)]
        for (L, rot, xd, w), y in zip(ins, ys):
            ref = C.host(_single(rot, xd, w, dt))
            assert np.array_equal(y.view(np.uint8), ref.view(np.uint8)), (L.spec, dt)
    # and against the oracle (the spec bar) for the float32 outputs
    ys = [C.host(y) for y in rl.paro_linear_batch(calls, out_dtype=torch.float32)]
    for (L, rot, xd, w), y in zip(ins, ys):
        deq = O.dequantize(*C.host_weights(w))
        if rot is None:
            ref = L.x.astype(np.float64) @ deq.T
        else:
            a = O.transform_activations(L.x, L.pairs, L.theta, L.scale)
            ref = O.f16_rne(a).astype(np.float64) @ deq.T
        mx, rel = C.linear_metrics(y, ref)
        assert mx <= C.MAX_ABS and rel <= C.REL_L2, (L.spec, mx, rel)


def test_batch_edge_cases():
    C.log("batch edge cases")
    ins = _batch_inputs([(80, 4, 256, 40, 2), (81, 1, 256, 8, None)])
    calls = [(rot, xd, *w) for (L, rot, xd, w) in ins]
    assert rl.paro_linear_batch([]) == []
    # an empty call inside a batch is skipped
    empty = (ins[0][1], torch.empty((0, 256), dtype=torch.float16, device="cuda"), *ins[0][3])
    ys = rl.paro_linear_batch([empty] + calls, out_dtype=torch.float32)
    assert ys[0].shape == (0, 40)
    for (L, rot, xd, w), y in zip(ins, ys[1:]):
        assert np.array_equal(C.host(y), C.host(_single(rot, xd, w, torch.float32)))
    # the same batch twice: identical bits
    a = [C.host(y) for y in rl.paro_linear_batch(calls)]
    b = [C.host(y) for y in rl.paro_linear_batch(calls)]
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint16), v.view(np.uint16))


@pytest.mark.parametrize("wid,Ms", [(2, (1, 4, 16)), (5, (64,))])
def test_workload_batch_as_benchmarked(wid, Ms):
    """The batched steps bench.py times, on the workload's own inputs: the attention projections
    q, k, v, o at M = 1, 4, 16 in one call (decode launches with the transform inside), and the
    8B-class layer's seven linears at M = 64 (batched transforms, grouped GEMM launches, one
    grouped split reduction). Every output is bit-identical to its single call and meets the
    spec bar against the oracle on sampled weight rows."""
    C.log(f"workload {wid} batch at M={Ms}")
    n_lin = {2: 4, 5: 7}[wid]
    ins = []
    for i in range(n_lin):
        L = C.linear_inputs(wid, i)
        rot = _rot(L)
        w = rl.paro_pack_weights(rot, C.dev(L.W, torch))
        for M in Ms:
            ins.append((L, rot, C.dev(L.x[:M], torch), w))
    calls = [(rot, xd, *w) for (L, rot, xd, w) in ins]
    ys = [C.host(y) for y in rl.paro_linear_batch(calls, out_dtype=torch.float32)]
    for (L, rot, xd, w), y in zip(ins, ys):
        single = C.host(rl.paro_rotated_linear(rot, xd, *w, out_dtype=torch.float32))
        assert np.array_equal(y.view(np.uint8), single.view(np.uint8)), (L.spec.name, xd.shape[0])
        rows = C.sample_rows(L.spec.N, 256, seed=xd.shape[0])
        deq = O.dequantize(*(t[rows] for t in C.host_weights(w)))
        a = O.transform_activations(L.x[:xd.shape[0]], L.pairs, L.theta, L.scale)
        ref = O.f16_rne(a).astype(np.float64) @ deq.T
        mx, rel = C.linear_metrics(y[:, rows], ref)
        assert mx <= C.MAX_ABS and rel <= C.REL_L2, (L.spec.name, xd.shape[0], mx, rel)
