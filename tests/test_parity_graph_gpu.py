"""paro_linear_batch captured in a HIP graph (torch.cuda.graph), as bench.py times it: the batches
that use the library's second stream (transforms of a second D beside the main D's; the long
calls' transforms run ahead with per-call ready events) join the capture through the fork event.
Each graph is replayed several times, with eager work of the program between the replays (the
outputs cleared, another eager batch, synchronizations), and every replay must give the eager
batch's bits."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
rl = pytest.importorskip("rotated_linear_amd")


def _calls(specs):
    out = []
    for seed, M, D, N, K in specs:
        L = W.custom_linear(seed, M, D, N, 0 if K is None else K)
        if K is None:
            rot, w = None, C.dev_weights(O.pack_weights(L.W, L.pairs[:0], L.theta[:0], np.ones_like(L.scale)), torch)
        else:
            rot = rl.paro_rotation_prepare(L.pairs, L.theta, L.scale)
            w = rl.paro_pack_weights(rot, C.dev(L.W, torch))
        out.append((rot, C.dev(L.x, torch), *w))
    return out


@pytest.mark.parametrize("specs", [
    # decode-shaped: two D (the second D's transforms on the side stream), 17..64-row calls in one
    # skinny launch with a split reduction, a plain call, an M <= 16 call on the decode kernel and
    # a single-row call of 8960 channels with its transform inside the decode kernel
    [(700, 64, 512, 256, 8), (701, 64, 512, 96, 8), (702, 40, 1024, 128, 8), (703, 64, 4224, 64, 8),
     (704, 33, 512, 64, None), (705, 8, 512, 64, 8), (706, 1, 8960, 96, 8)],
    # prefill-shaped: three long rotated calls (transforms ahead on the side stream, ready events),
    # a long plain call and a short rotated call
    [(710, 300, 512, 96, 8), (711, 257, 1024, 64, 2), (712, 400, 512, 128, 12), (713, 300, 512, 64, None),
     (714, 40, 512, 64, 8)],
])
def test_captured_batch_replays_match_eager(specs):
    C.log(f"captured batch of {len(specs)} calls")
    calls = _calls(specs)
    # at least the batch's workspace (the calls' workspaces one after another)
    need = sum(rl.paro_workspace_bytes(x.shape[0], x.shape[1], q.shape[0]) for (_, x, q, _, _) in calls)
    outs_e = [torch.empty((x.shape[0], q.shape[0]), dtype=torch.float16, device="cuda") for (_, x, q, _, _) in calls]
    outs_g = [torch.empty_like(y) for y in outs_e]
    ws_e = torch.empty(max(need, 1 << 20), dtype=torch.uint8, device="cuda")
    ws_g = torch.empty_like(ws_e)
    # eager first (it also creates the library's second stream, outside any capture)
    rl.paro_linear_batch(calls, outs=outs_e, ws=ws_e)
    torch.cuda.synchronize()
    ref = [C.host(y) for y in outs_e]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        rl.paro_linear_batch(calls, outs=outs_g, ws=ws_g)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rl.paro_linear_batch(calls, outs=outs_g, ws=ws_g)
    torch.cuda.synchronize()
    for rep in range(3):
        for y in outs_g:
            y.zero_()
        ws_g.zero_()
        rl.paro_linear_batch(calls, outs=outs_e, ws=ws_e)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (y, r) in enumerate(zip(outs_g, ref)):
            assert np.array_equal(C.host(y).view(np.uint16), r.view(np.uint16)), (rep, i, specs[i])
        for i, (y, r) in enumerate(zip(outs_e, ref)):
            assert np.array_equal(C.host(y).view(np.uint16), r.view(np.uint16)), ("eager", rep, i)
    del g
