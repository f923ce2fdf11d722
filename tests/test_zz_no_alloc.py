"""paro_rotated_linear_noalloc: the workspace-free variant of paro_rotated_linear, for callers that
cannot allocate device memory. Its workspace is the library's fixed scratch array, so it must give
exactly what paro_rotated_linear gives with a caller-owned workspace (same kernels, same split of
the reduction, same summation order), call after call, with the scratch keeping whatever the
previous call left in it; and it must meet the linear's bar against the oracle."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
rl = pytest.importorskip("rotated_linear_amd")


def _case(seed, M, D, N, K):
    L = W.custom_linear(seed, M, D, N, K)
    rot = rl.paro_rotation_prepare(L.pairs, L.theta, L.scale)
    w = rl.paro_pack_weights(rot, C.dev(L.W, torch))
    return L, rot, w


def _check(L, rot, w, dt):
    M, N = L.x.shape[0], L.spec.N
    xd = C.dev(L.x, torch)
    need = rl.paro_workspace_bytes(M, L.spec.D, N)
    assert need <= rl.paro_noalloc_max_bytes()
    out = torch.empty((M, N), dtype=dt, device="cuda")
    got = C.host(rl.paro_rotated_linear_noalloc(rot, xd, *w, out=out))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    ref_call = C.host(rl.paro_rotated_linear(rot, xd, *w, out_dtype=dt, ws=ws))
    assert np.array_equal(got.view(np.uint8), ref_call.view(np.uint8)), "differs from paro_rotated_linear"
    if dt == torch.float32:
        deq = O.dequantize(*C.host_weights(w))
        a = O.transform_activations(L.x, L.pairs, L.theta, L.scale)
        mx, rel = C.linear_metrics(got, O.f16_rne(a).astype(np.float64) @ deq.T)
        assert mx <= C.MAX_ABS and rel <= C.REL_L2, (mx, rel)


@pytest.mark.parametrize("dt", [torch.float32, torch.float16])
def test_noalloc_matches_workspace_call_twice(dt):
    """Two calls in a row through the scratch, the second smaller (the scratch then holds the first
    call's larger leftovers), each bit-identical to the workspace call and within the oracle bar;
    then decode-shaped calls (transform inside the decode kernel: no scratch), one of them a single
    row of 8960 channels."""
    big = _case(1301, 300, 4096, 1024, 8)  # transform kernel + GEMM with split partials in the scratch
    small = _case(1302, 40, 1024, 200, 8)
    dec = _case(1303, 4, 1536, 512, 8)
    wide = _case(1305, 1, 8960, 256, 8)
    for name, (L, rot, w) in (("M=300 D=4096 N=1024", big), ("M=40 D=1024 N=200", small),
                              ("M=4 D=1536 N=512", dec), ("M=1 D=8960 N=256", wide),
                              ("M=300 D=4096 N=1024 again", big)):
        C.log(f"noalloc {name} {dt}")
        _check(L, rot, w, dt)


def test_noalloc_rejects_what_does_not_fit():
    """A call whose workspace exceeds the scratch returns PARO_EWORKSPACE before anything is
    enqueued (down_proj-sized prefill: 4096 rows of 14336 channels need 117 MB for x')."""
    D, M, N = 14336, 4096, 128
    assert rl.paro_workspace_bytes(M, D, N) > rl.paro_noalloc_max_bytes()
    L = W.custom_linear(1304, 1, D, N, 2)
    rot = rl.paro_rotation_prepare(L.pairs, L.theta, L.scale)
    w = rl.paro_pack_weights(rot, C.dev(L.W, torch))
    x = torch.zeros((M, D), dtype=torch.float16, device="cuda")
    out = torch.full((M, N), 3.0, dtype=torch.float16, device="cuda")
    with pytest.raises(rl.ParoError, match="EWORKSPACE"):
        rl.paro_rotated_linear_noalloc(rot, x, *w, out=out)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "nothing may be written on an error"
