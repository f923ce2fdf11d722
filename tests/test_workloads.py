"""CPU tests of the seeded input generators (no arithmetic of the method lives there)."""
import numpy as np

import workloads as W


def test_deterministic_and_shapes():
    a = W.make_linear(2, 1)
    b = W.make_linear(2, 1)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.W, b.W)
    assert np.array_equal(a.pairs, b.pairs) and np.array_equal(a.theta, b.theta)
    assert a.x.shape == (16, 1536) and a.W.shape == (256, 1536)
    assert a.pairs.shape == (8, 768, 2) and a.theta.shape == (8, 768) and a.scale.shape == (1536,)
    assert a.x.dtype == np.float16 and a.W.dtype == np.float16
    assert a.pairs.dtype == np.int32 and a.theta.dtype == np.float32 and a.scale.dtype == np.float32


def test_linears_independent_and_prefix_batches():
    q = W.make_linear(2, 0)
    k = W.make_linear(2, 1)
    assert not np.array_equal(q.pairs, k.pairs)
    small = W.make_linear(2, 0, M=4)
    assert np.array_equal(small.x, q.x[:4])


def test_recipe_properties():
    L = W.make_linear(2, 0)
    for k in range(L.pairs.shape[0]):
        assert np.array_equal(np.sort(L.pairs[k].ravel()), np.arange(1536))
    assert np.all(L.scale > 0) and np.all(np.abs(L.theta) <= np.pi)
    # 0.5% activation outlier channels x30: their column RMS stands out
    rms = np.sqrt((L.x.astype(np.float64) ** 2).mean(axis=0))
    assert int((rms > 10).sum()) == round(0.005 * 1536)
    t = W.make_linear(1)
    assert t.x.shape == (4, 256) and t.W.shape == (512, 256) and t.pairs.shape == (2, 128, 2)
    assert np.all(np.abs(t.x[:, [3, 77]]).mean() > 5)


def test_custom_shapes():
    c = W.custom_linear(7, 5, 384, 200, 3)
    assert c.x.shape == (5, 384) and c.W.shape == (200, 384) and c.pairs.shape == (3, 192, 2)
    z = W.custom_linear(7, 1, 256, 8, 0)
    assert z.pairs.shape == (0, 128, 2) and z.theta.shape == (0, 128)


def test_model_stack():
    assert W.MODEL_LAYERS == 28 and len(W.MODEL_LINEARS) == 7
    assert sorted(i for ph in W.MODEL_PHASES for i in ph) == list(range(7))
    a = W.make_model_linear(3, 6, with_weights=False)
    b = W.make_model_linear(4, 6, with_weights=False)
    assert a.x.shape == (1, 8960) and a.pairs.shape == (8, 4480, 2) and a.W.shape == (0, 8960)
    assert not np.array_equal(a.pairs, b.pairs)  # every layer has its own transform
    g = W.make_model_linear(0, 4)
    assert g.W.shape == (8960, 1536) and g.x.shape == (1, 1536)
    assert np.array_equal(W.make_model_linear(0, 4, with_weights=False).pairs, g.pairs)
