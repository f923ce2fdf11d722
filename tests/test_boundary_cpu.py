"""CPU tests of the C-ABI boundary: the library loads, exports every declared entry
point, and rejects bad arguments on the host before any HIP call is made.

Pointers handed to the library here are fake (never dereferenced): every case
returns from host-side validation before anything is enqueued.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paro.h")

rl = pytest.importorskip("rotated_linear_amd", reason="libparo.so not built")
lib = rl.lib()
P = ctypes.POINTER(rl.paro_rotation)
FAKE = 0x100000  # 16-byte aligned, never dereferenced on these paths


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(paro_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) == 14, names
    out = subprocess.run(["nm", "-D", "--defined-only", rl.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(paro_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(lib, n)
    assert set(names) == set(rl.EXPORTS)


def test_status_strings_and_sizes():
    for s in range(7):
        assert lib.paro_status_str(s).decode().startswith(rl.STATUS[s])
    assert lib.paro_status_str(99) == b"PARO_UNKNOWN"
    assert lib.paro_version() >= 100
    # descriptor: one 12-byte record (pair word, cos, sin) per pair per stage + 1/s and s (4 B each)
    # per channel, each section padded to 256 bytes
    assert rl.paro_rotation_bytes(8, 1536) == 8 * 768 * 12 + 2 * 1536 * 4
    assert rl.paro_rotation_bytes(0, 128) == 2 * 512
    for K, D in ((8, 100), (8, 1537), (-1, 256), (65, 256), (2, 16512), (2, 0)):
        assert rl.paro_rotation_bytes(K, D) == 0, (K, D)
    assert rl.paro_workspace_bytes(1, 1536, 1536) == 1536 * 2  # an upper bound: the fused path uses none
    # prefill-shaped: the transformed x, then room for the GEMM's split partial sums (float32)
    ws = rl.paro_workspace_bytes(64, 4096, 4096)
    assert ws >= 64 * 4096 * 2 and ws % 256 == 0
    assert ws <= 64 * 4096 * 2 + 16 * 64 * 4096 * 4
    assert rl.paro_workspace_bytes(0, 4096, 4096) == 0


def _prep(K, D, pairs, theta, scale, desc=FAKE, nbytes=1 << 30, out=True):
    h = rl.paro_rotation()
    return lib.paro_rotation_prepare(K, D, pairs.ctypes.data_as(ctypes.c_void_p) if pairs is not None else None,
                                     theta.ctypes.data_as(ctypes.c_void_p) if theta is not None else None,
                                     scale.ctypes.data_as(ctypes.c_void_p) if scale is not None else None,
                                     desc, nbytes, ctypes.byref(h) if out else None, None)


def _good(K=2, D=256, seed=0):
    rng = np.random.default_rng(seed)
    pairs = np.stack([rng.permutation(D).reshape(D // 2, 2) for _ in range(K)]).astype(np.int32)
    theta = rng.uniform(-3, 3, (K, D // 2)).astype(np.float32)
    scale = np.exp(rng.normal(0, 0.3, D)).astype(np.float32)
    return pairs, theta, scale


def test_prepare_rejects_bad_matchings():
    pairs, theta, scale = _good()
    dup = pairs.copy()
    dup[1, 5, 0] = dup[1, 6, 1]  # channel used twice in stage 1, another one missing
    assert _prep(2, 256, dup, theta, scale) == 3
    oor = pairs.copy()
    oor[0, 0, 1] = 256
    assert _prep(2, 256, oor, theta, scale) == 3
    neg = pairs.copy()
    neg[0, 3, 0] = -1
    assert _prep(2, 256, neg, theta, scale) == 3
    self_pair = pairs.copy()
    self_pair[0, 0, 1] = self_pair[0, 0, 0]
    assert _prep(2, 256, self_pair, theta, scale) == 3


def test_prepare_rejects_bad_scales_and_angles():
    pairs, theta, scale = _good()
    for bad in (0.0, -1.0, np.inf, np.nan):
        s = scale.copy()
        s[17] = bad
        assert _prep(2, 256, pairs, theta, s) == 4, bad
    t = theta.copy()
    t[1, 3] = np.nan
    assert _prep(2, 256, pairs, t, scale) == 4
    s = scale.copy()
    s[0] = 1e-45  # 1/s overflows float32
    assert _prep(2, 256, pairs, theta, s) == 4


def test_prepare_rejects_bad_shapes_and_pointers():
    pairs, theta, scale = _good()
    assert _prep(2, 200, pairs, theta, scale) == 2
    assert _prep(2, 255, pairs, theta, scale) == 2
    assert _prep(65, 256, pairs, theta, scale) == 2
    assert _prep(2, 256, pairs, theta, scale, desc=None) == 1
    assert _prep(2, 256, pairs, theta, scale, desc=FAKE + 8) == 1  # misaligned
    assert _prep(2, 256, pairs, theta, scale, nbytes=100) == 1  # descriptor too small
    assert _prep(2, 256, pairs, theta, scale, out=False) == 1
    assert _prep(2, 256, None, theta, scale) == 1


def _rot(K=2, D=256, dev=FAKE):
    return rl.paro_rotation(K, D, dev)


def test_calls_reject_bad_arguments_before_launch():
    r = _rot()
    v = ctypes.c_void_p
    # pack
    assert lib.paro_pack_weights(None, 4, v(FAKE), v(FAKE * 2), v(FAKE * 3), v(FAKE * 4), None) == 1
    assert lib.paro_pack_weights(ctypes.byref(r), -1, v(FAKE), v(FAKE * 2), v(FAKE * 3), v(FAKE * 4), None) == 1
    assert lib.paro_pack_weights(ctypes.byref(r), 0, None, None, None, None, None) == 0  # nothing to do
    assert lib.paro_pack_weights(ctypes.byref(r), 4, v(FAKE), v(FAKE), v(FAKE * 3), v(FAKE * 4), None) == 1  # alias
    bad_shape = _rot(2, 250)
    assert lib.paro_pack_weights(ctypes.byref(bad_shape), 4, v(FAKE), v(FAKE * 2), v(FAKE * 3), v(FAKE * 4), None) == 2
    misaligned = _rot(2, 256, FAKE + 4)
    assert lib.paro_rotate(ctypes.byref(misaligned), 4, v(FAKE), v(FAKE * 2), None) == 1
    # rotate
    assert lib.paro_rotate(ctypes.byref(r), 0, None, None, None) == 0
    assert lib.paro_rotate(ctypes.byref(r), -2, v(FAKE), v(FAKE * 2), None) == 1
    assert lib.paro_rotate(ctypes.byref(r), 4, v(FAKE), v(FAKE + 256), None) == 1  # overlapping in/out
    assert lib.paro_rotate(ctypes.byref(r), 4, v(FAKE + 2), v(FAKE * 2), None) == 1  # misaligned
    # plain linear
    args = (v(FAKE), v(FAKE * 2), v(FAKE * 3), v(FAKE * 4))
    assert lib.paro_w4a16_linear(4, 256, 64, *args, v(FAKE * 5), 7, None, 0, None) == 1  # dtype
    assert lib.paro_w4a16_linear(4, 250, 64, *args, v(FAKE * 5), 0, None, 0, None) == 2  # D
    assert lib.paro_w4a16_linear(4, 256, 64, *args, v(FAKE), 0, None, 0, None) == 1  # y aliases x
    assert lib.paro_w4a16_linear(0, 256, 64, *args, v(FAKE * 5), 0, None, 0, None) == 0  # empty
    assert lib.paro_w4a16_linear(4, 256, 0, *args, v(FAKE * 5), 0, None, 0, None) == 0  # empty
    assert lib.paro_w4a16_linear(-1, 256, 64, *args, v(FAKE * 5), 0, None, 0, None) == 1
    assert lib.paro_w4a16_linear(4, 256, 64, None, *args[1:], v(FAKE * 5), 0, None, 0, None) == 1
    assert lib.paro_w4a16_linear(4, 256, 64, *args[:2], v(FAKE * 3 + 1), args[3], v(FAKE * 5), 0, None, 0,
                                 None) == 1  # odd scales pointer
    # rotated linear: large M needs a workspace
    big = _rot(8, 4096)
    assert rl.paro_workspace_bytes(64, 4096, 512) > 0
    assert lib.paro_rotated_linear(ctypes.byref(big), 64, 512, *args, v(FAKE * 5), 0, None, 0, None) == 5
    assert lib.paro_rotated_linear(ctypes.byref(big), 64, 512, *args, v(FAKE * 5), 0, v(FAKE * 6), 100, None) == 5
    assert lib.paro_rotated_linear(None, 1, 512, *args, v(FAKE * 5), 0, None, 0, None) == 1
    # the workspace is written: it may overlap no operand and not the descriptor
    need = rl.paro_workspace_bytes(64, 4096, 512)
    assert lib.paro_rotated_linear(ctypes.byref(big), 64, 512, *args, v(FAKE * 5), 0, v(FAKE * 2), need, None) == 1
    assert lib.paro_rotated_linear(ctypes.byref(big), 64, 512, *args, v(FAKE * 5), 0, v(FAKE * 4), need, None) == 1
    far = _rot(8, 4096, FAKE * 40)
    assert lib.paro_rotated_linear(ctypes.byref(far), 64, 512, *args, v(FAKE * 5), 0, v(FAKE * 40), need, None) == 1
    plain_need = rl.paro_workspace_bytes(64, 4096, 512) - 64 * 4096 * 2
    assert lib.paro_w4a16_linear(64, 4096, 512, *args, v(FAKE * 5), 0, v(FAKE * 3), plain_need, None) == 1


def _call(rot, M, D, N, base):
    """A batch entry with fake, non-overlapping buffers starting at FAKE * base."""
    v = FAKE * base
    return rl.paro_linear_args(ctypes.pointer(rot) if rot is not None else None, M, D, N, v, v + FAKE // 2,
                               v + FAKE // 2 + FAKE // 4, v + FAKE // 2 + FAKE // 4 + FAKE // 8, v + FAKE)


def test_batch_rejects_bad_arguments_before_launch():
    Arr = rl.paro_linear_args * 4
    ok = _rot(8, 256)
    # nothing to do
    assert lib.paro_linear_batch(0, None, 0, None, 0, None) == 0
    assert lib.paro_linear_batch(-1, None, 0, None, 0, None) == 1
    assert lib.paro_linear_batch(2, None, 0, None, 0, None) == 1
    a = Arr(_call(ok, 4, 256, 64, 4), _call(None, 4, 256, 64, 8))
    assert lib.paro_linear_batch(2, a, 7, None, 0, None) == 1  # dtype
    a = Arr(_call(ok, 4, 512, 64, 4))  # D differs from the transform's
    assert lib.paro_linear_batch(1, a, 0, None, 0, None) == 1
    a = Arr(_call(None, 4, 250, 64, 4))
    assert lib.paro_linear_batch(1, a, 0, None, 0, None) == 2
    a = Arr(_call(_rot(8, 250), 4, 250, 64, 4))
    assert lib.paro_linear_batch(1, a, 0, None, 0, None) == 2
    # one call's output overlaps another call's input
    c0, c1 = _call(ok, 4, 256, 64, 4), _call(None, 4, 256, 64, 8)
    c1.x = c0.y
    a = Arr(c0, c1)
    assert lib.paro_linear_batch(2, a, 0, None, 0, None) == 1
    c1 = _call(None, 4, 256, 64, 8)
    c1.y = c0.y
    a = Arr(c0, c1)
    assert lib.paro_linear_batch(2, a, 0, None, 0, None) == 1
    # a transform the decode kernel does not take needs a workspace
    deep = _rot(12, 256)
    a = Arr(_call(deep, 4, 256, 64, 4), _call(ok, 4, 256, 64, 8))
    need = lib.paro_linear_batch_workspace_bytes(2, a)
    assert need == 4 * 256 * 2
    assert lib.paro_linear_batch(2, a, 0, None, 0, None) == 5
    assert lib.paro_linear_batch(2, a, 0, ctypes.c_void_p(FAKE * 12), need - 1, None) == 5
    assert lib.paro_linear_batch(2, a, 0, ctypes.c_void_p(FAKE * 4), need, None) == 1  # workspace overlaps x
    wq = a[1].qweight  # ... or another call's packed weights, or a transform's descriptor
    assert lib.paro_linear_batch(2, a, 0, ctypes.c_void_p(wq), need, None) == 1
    a = Arr(_call(_rot(12, 256, FAKE * 30), 4, 256, 64, 4), _call(ok, 4, 256, 64, 8))
    assert lib.paro_linear_batch(2, a, 0, ctypes.c_void_p(FAKE * 30), need, None) == 1
    big = _rot(8, 4096)
    a = Arr(_call(big, 64, 4096, 64, 4))
    need = lib.paro_linear_batch_workspace_bytes(1, a)
    assert 64 * 4096 * 2 <= need <= rl.paro_workspace_bytes(64, 4096, 64)
    assert lib.paro_linear_batch_workspace_bytes(0, a) == 0


# --------------------------------------------------------------------------- #
# descriptor encoding and the bank-conflict-free pair order (host only)
# --------------------------------------------------------------------------- #

def _encode(pairs, theta, scale):
    K, D = pairs.shape[0], scale.shape[0]
    return rl.descriptor_sections(rl.paro_rotation_encode(pairs, theta, scale), K, D)


@pytest.mark.parametrize("D,K", [(128, 1), (256, 2), (1536, 8), (8960, 2), (16384, 1)])
def test_schedule_is_conflict_free_and_same_rotation(D, K):
    import math
    pairs, theta, scale = _good(K, D, seed=D)
    ep, ecs, inv_s, s = _encode(pairs, theta, scale)
    assert np.array_equal(s, scale)
    assert np.array_equal(inv_s, (1.0 / scale.astype(np.float64)).astype(np.float32))
    for k in range(K):
        # same set of rotations: (i, j, c, s) or (j, i, c, -s)
        want = {}
        for (i, j), t in zip(pairs[k], theta[k]):
            c = np.float32(math.cos(float(t)))
            sn = np.float32(math.sin(float(t)))
            want[(int(i), int(j))] = (c, sn)
        for (i, j), (c, sn) in zip(ep[k], ecs[k]):
            if (int(i), int(j)) in want:
                assert want[(int(i), int(j))] == (c, sn)
            else:
                wc, ws = want[(int(j), int(i))]
                assert wc == c and ws == -sn
        assert len(want) == D // 2
        # every aligned run of q pairs has distinct first and second channels mod q
        for q in (64, 32, 16, 8):
            ii = (ep[k, :, 0] % q).reshape(-1, q)
            jj = (ep[k, :, 1] % q).reshape(-1, q)
            assert all(len(set(r)) == q for r in ii), (q, "first channels collide")
            assert all(len(set(r)) == q for r in jj), (q, "second channels collide")


def test_schedule_depends_only_on_the_pair_set():
    pairs, theta, scale = _good(3, 1024, seed=4)
    base = rl.paro_rotation_encode(pairs, theta, scale)
    rng = np.random.default_rng(1)
    p2, t2 = pairs.copy(), theta.copy()
    for k in range(3):
        perm = rng.permutation(512)
        p2[k], t2[k] = p2[k][perm], t2[k][perm]
    assert np.array_equal(rl.paro_rotation_encode(p2, t2, scale), base)


def test_encode_errors_match_prepare():
    pairs, theta, scale = _good()
    bad = pairs.copy()
    bad[0, 1] = bad[0, 0]
    with pytest.raises(rl.ParoError) as e:
        rl.paro_rotation_encode(bad, theta, scale)
    assert e.value.status == 3
    s = scale.copy()
    s[3] = -2
    with pytest.raises(rl.ParoError) as e:
        rl.paro_rotation_encode(pairs, theta, s)
    assert e.value.status == 4


def test_import_fails_loudly_without_the_library(tmp_path):
    """No CPU fallback: a copy of the package without libparo.so refuses to import."""
    import shutil
    import subprocess
    import sys

    pkg = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "rotated_linear_amd")
    dst = tmp_path / "rotated_linear_amd"
    dst.mkdir()
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            shutil.copy(os.path.join(pkg, f), dst / f)
    r = subprocess.run([sys.executable, "-c", "import rotated_linear_amd"], cwd=tmp_path, capture_output=True,
                       text=True, env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libparo.so is missing" in r.stderr


def test_binding_checks_outputs_and_workspaces_before_launch():
    """The binding checks every output and workspace tensor (shape, dtype, contiguity) as it does
    the inputs, before any library call: an undersized or strided buffer would otherwise be
    written past its end on the device. Here every tensor lives on the CPU, so a call that got
    past the checks would stop at the device check ("must live on the GPU")."""
    import torch

    D, N, M = 256, 40, 3
    rot = rl.Rotation(2, D, None, rl.paro_rotation(2, D, FAKE))
    x = torch.zeros((M, D), dtype=torch.float16)
    qw = torch.zeros((N, D // 2), dtype=torch.uint8)
    sc = torch.zeros((N, D // 128), dtype=torch.float16)
    z = torch.zeros((N, D // 128), dtype=torch.float16)
    good_out = torch.zeros((M, N), dtype=torch.float16)

    def raises(fn, kind, text):
        with pytest.raises(kind, match=text):
            fn()

    for call in (lambda **k: rl.paro_w4a16_linear(x, qw, sc, z, **k),
                 lambda **k: rl.paro_rotated_linear(rot, x, qw, sc, z, **k)):
        raises(lambda: call(out=torch.zeros((M, N - 1), dtype=torch.float16)), ValueError, "out must have shape")
        raises(lambda: call(out=torch.zeros((M + 1, N), dtype=torch.float16)), ValueError, "out must have shape")
        raises(lambda: call(out=torch.zeros((N, M), dtype=torch.float16).t()), ValueError, "contiguous")
        raises(lambda: call(out=torch.zeros((M, N), dtype=torch.bfloat16)), TypeError, "float16 or float32")
        raises(lambda: call(out=good_out, out_dtype=torch.float32), TypeError, "out must be")
        raises(lambda: call(out=good_out, ws=torch.zeros(512, dtype=torch.float32)), TypeError, "ws must be")
        raises(lambda: call(out=good_out, ws=torch.zeros((2, 256), dtype=torch.uint8)), ValueError, "ws must have")
        raises(lambda: call(out=good_out, ws=torch.zeros(1024, dtype=torch.uint8)[::2]), ValueError, "contiguous")
        raises(lambda: call(out=good_out), ValueError, "must live on the GPU")
    raises(lambda: rl.paro_rotate(rot, x, out=torch.zeros((M, D - 2), dtype=torch.float16)), ValueError,
           "out must have shape")
    raises(lambda: rl.paro_rotate(rot, x, out=torch.zeros((M, D), dtype=torch.float32)), TypeError, "out must be")
    W = torch.zeros((N, D), dtype=torch.float16)
    raises(lambda: rl.paro_pack_weights(rot, W, out=(qw[:-1], sc, z)), ValueError, "qweight must have shape")
    raises(lambda: rl.paro_pack_weights(rot, W, out=(qw, sc.float(), z)), TypeError, "scales must be")
    raises(lambda: rl.paro_pack_weights(rot, W, out=(qw, sc, z[:, :1])), ValueError, "zeros must have shape")
    raises(lambda: rl.paro_pack_weights(rot, W, out=(qw, sc, z)), ValueError, "must live on the GPU")
    calls = [(rot, x, qw, sc, z), (None, x, qw, sc, z)]
    raises(lambda: rl.paro_linear_batch(calls, outs=[good_out]), ValueError, "outs has 1 tensors")
    raises(lambda: rl.paro_linear_batch(calls, outs=[good_out, torch.zeros((M, N + 1), dtype=torch.float16)]),
           ValueError, "out must have shape")
    raises(lambda: rl.paro_linear_batch(calls, outs=[good_out, good_out.float()]), TypeError, "out must be")
    raises(lambda: rl.paro_linear_batch(calls, ws=torch.zeros(64, dtype=torch.int8)), TypeError, "ws must be")
    raises(lambda: rl.paro_linear_batch(calls, outs=[good_out, good_out.clone()]), ValueError, "must live on the GPU")
