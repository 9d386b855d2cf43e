"""Pins of the oracle's layer steps (short convolution, activations, norms,
gates) to facts other than their own formulas (CPU only)."""
import numpy as np

from oracle import layer as L


def test_conv_hand_example():
    """Width-4 causal convolution, weight index 0 on t-3 and 3 on t, no cache:
    y = [0.4*1, 0.3*1 + 0.4*2, 0.2*1 + 0.3*2 + 0.4*3, 0.1*1 + 0.2*2 + 0.3*3 + 0.4*4]."""
    x = np.array([1.0, 2.0, 3.0, 4.0]).reshape(4, 1, 1)
    w = np.array([0.1, 0.2, 0.3, 0.4]).reshape(1, 1, 4)
    y, c = L.short_conv(x, w)
    assert np.allclose(y.ravel(), [0.4, 1.1, 2.0, 3.0], atol=1e-15)
    assert np.array_equal(c.ravel(), [2.0, 3.0, 4.0])   # the last three inputs


def test_conv_equals_library_convolution():
    rng = np.random.default_rng(0)
    T, H, d = 37, 2, 3
    x = rng.standard_normal((T, H, d))
    w = rng.standard_normal((H, d, 4))
    y, _ = L.short_conv(x, w)
    for h in range(H):
        for c in range(d):
            ref = np.convolve(x[:, h, c], w[h, c, ::-1])[:T]
            assert np.allclose(y[:, h, c], ref, atol=1e-13)


def test_conv_cache_continuation_and_short_calls():
    rng = np.random.default_rng(1)
    T, H, d = 20, 2, 4
    x = rng.standard_normal((T, H, d))
    w = rng.standard_normal((H, d, 4))
    c0 = rng.standard_normal((3, H, d))
    y_all, c_all = L.short_conv(x, w, c0)
    # any split, including pieces shorter than the window
    for cuts in ([7], [1, 2], [2, 3, 4, 19], [19]):
        bounds = [0] + cuts + [T]
        c, ys = c0, []
        for s, e in zip(bounds[:-1], bounds[1:]):
            y, c = L.short_conv(x[s:e], w, c)
            ys.append(y)
        assert np.allclose(np.concatenate(ys), y_all, atol=1e-13)
        assert np.array_equal(c, c_all)
    # cache = the three inputs before the next token
    ext = np.concatenate([c0, x])
    assert np.array_equal(c_all, ext[-3:])


def test_activation_and_gate_values():
    assert L.silu(0.0) == 0.0
    assert np.isclose(L.silu(1.0), 1.0 / (1.0 + np.exp(-1.0)), rtol=0, atol=1e-16)
    assert np.isclose(L.silu(40.0), 40.0) and abs(L.silu(-40.0)) < 1e-15
    a = np.linspace(-30, 30, 61)
    la = L.G_MIN * L.sigmoid(a)
    assert np.all(la < 0) and np.all(la > -5) and np.isclose(L.G_MIN * L.sigmoid(0.0), -2.5)
    assert L.sigmoid(0.0) == 0.5


def test_l2norm_unit_vectors():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 3, 128)) * 10
    n = np.linalg.norm(L.l2norm(x), axis=-1)
    s = np.linalg.norm(x, axis=-1)
    assert np.allclose(n, s / np.sqrt(s * s + L.L2_EPS), rtol=1e-14)
    assert np.allclose(n, 1.0, atol=1e-8)


def test_epilogue_hand_example_and_invariance():
    # d = 2: o = (3, 4), mean square 12.5
    o = np.array([[3.0, 4.0]])
    w = np.array([2.0, 0.5])
    g = np.array([[0.0, 100.0]])          # gates 1/2 and 1
    out = L.epilogue(o, g, w, eps=0.0)
    r = np.sqrt(12.5)
    assert np.allclose(out, [[3 / r * 2 * 0.5, 4 / r * 0.5 * 1.0]], atol=1e-15)
    rng = np.random.default_rng(3)
    o = rng.standard_normal((4, 2, 128))
    g = rng.standard_normal((4, 2, 128))
    w = rng.standard_normal(128)
    assert np.allclose(L.epilogue(7.5 * o, g, w, eps=0.0), L.epilogue(o, g, w, eps=0.0), atol=1e-13)
    # unit weight, open gate: RMS of the output is 1
    out = L.epilogue(o, np.full_like(o, 60.0), np.ones(128), eps=0.0)
    assert np.allclose(np.sqrt(np.mean(out * out, axis=-1)), 1.0, atol=1e-12)


def test_prologue_composition():
    """q and k come out unit-norm, v is silu of the convolution, the cache
    holds the raw inputs."""
    rng = np.random.default_rng(4)
    T, H, d = 9, 2, 128
    raw = [rng.standard_normal((T, H, d)) for _ in range(3)]
    cw = rng.standard_normal((3, H, d, 4)) * 0.5
    a, b = rng.standard_normal((T, H, d)), rng.standard_normal((T, H))
    q, k, v, la, be, c = L.prologue(*raw, cw, a, b)
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-6)
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-6)
    y, _ = L.short_conv(raw[2], cw[2])
    assert np.allclose(v, y / (1 + np.exp(-y)), atol=1e-14)
    assert np.array_equal(c[1], raw[1][-3:])
    assert la.shape == (T, H, d) and be.shape == (T, H)


def test_prologue_gate_outputs_pinned():
    """log alpha = -5 sigmoid(a) and beta = sigmoid(b), read out of prologue()
    itself at points where the values are fixed without the formula: a = 0
    gives the midpoint -2.5, a -> +inf the lower bound -5, a -> -inf no
    decay (0); b = 0 gives 1/2, b -> +inf full write (1), b -> -inf none (0).
    ("Kimi K3 技术报告解读" section 3.3 class KDA and section 3.5: the decay's
    log is bounded below by g_min = -5 through a sigmoid; the write gate is a
    sigmoid.)  A sign error (sigmoid(-a) or sigmoid(-b)) swaps the limits."""
    T, H, d = 3, 2, 128
    raw = [np.zeros((T, H, d)) for _ in range(3)]
    cw = np.zeros((3, H, d, 4))
    a = np.zeros((T, H, d))
    a[1] = 60.0
    a[2] = -60.0
    b = np.array([[0.0, 0.0], [60.0, 60.0], [-60.0, -60.0]])
    _, _, _, la, be, _ = L.prologue(*raw, cw, a, b)
    assert np.array_equal(la[0], np.full((H, d), -2.5))
    assert np.allclose(la[1], -5.0, rtol=0, atol=1e-24)
    assert np.all(la[2] <= 0) and np.all(la[2] > -1e-24)
    assert np.array_equal(be[0], np.full(H, 0.5))
    assert np.allclose(be[1], 1.0, rtol=0, atol=1e-24)
    assert np.all(be[2] >= 0) and np.all(be[2] < 1e-24)
    # strictly monotone in the same direction as the pre-activation
    a = np.linspace(-8, 8, 17)[:, None, None] * np.ones((1, H, d))
    b = np.linspace(-8, 8, 17)[:, None] * np.ones((1, H))
    raw = [np.zeros((17, H, d)) for _ in range(3)]
    _, _, _, la, be, _ = L.prologue(*raw, cw, a, b)
    assert np.all(np.diff(la[:, 0, 0]) < 0) and np.all(np.diff(be[:, 0]) > 0)
