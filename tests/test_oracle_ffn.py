"""Pins of the oracle's FFN epilogues (squared ReLU, gated squared ReLU, dReLU).

Pins: the elementwise closed forms, and whole FFNs on integer-valued tiny
inputs against brute-force loops (exact), including the second top-K on the
intermediate and the nonzero gather of the dReLU down projection.
"""
import itertools

import numpy as np

import oracle


def test_relu2_closed_form():
    u = np.array([-2.0, -0.0, 0.0, 0.5, 3.0, -1e-300])
    assert oracle.relu2(u).tolist() == [0.0, 0.0, 0.0, 0.25, 9.0, 0.0]


def test_relu2_glu_closed_form_and_sign():
    g = np.array([-2.0, 0.0, 0.5, 3.0, 3.0, 2.0])
    u = np.array([5.0, 7.0, 4.0, -1.0, 0.0, 0.25])
    assert oracle.relu2_glu(g, u).tolist() == [0.0, 0.0, 1.0, -9.0, 0.0, 1.0]
    rng = np.random.default_rng(5)
    g = rng.integers(-4, 5, size=300).astype(np.float64)
    u = rng.integers(-4, 5, size=300).astype(np.float64)
    h = oracle.relu2_glu(g, u)
    # zero wherever the gate is not positive; the sign of h is the sign of up
    assert np.all(h[g <= 0] == 0)
    assert np.array_equal(np.sign(h), np.where(g > 0, np.sign(u), 0.0))
    # with up equal to the gate it is relu(g)^3, i.e. relu2(g) * g
    assert np.array_equal(oracle.relu2_glu(g, g), oracle.relu2(g) * g)


def test_drelu_closed_form_and_support():
    g = np.array([-1.0, 2.0, 0.0, 3.0, -4.0])
    u = np.array([5.0, -1.0, 7.0, 2.0, -2.0])
    h = oracle.drelu(g, u)
    assert h.tolist() == [0.0, 0.0, 0.0, 6.0, 0.0]
    rng = np.random.default_rng(1)
    g = rng.integers(-3, 4, size=200).astype(np.float64)
    u = rng.integers(-3, 4, size=200).astype(np.float64)
    h = oracle.drelu(g, u)
    assert np.array_equal(h != 0, (g > 0) & (u > 0))
    assert np.array_equal(h, np.where((g > 0) & (u > 0), g * u, 0.0))


def _topk_loop(vals, k):
    order = sorted(range(len(vals)), key=lambda j: (-abs(vals[j]), j))
    return set(order[:k])


def test_ffn_relu2_brute_force():
    rng = np.random.default_rng(2)
    d, f = 9, 7
    x = rng.integers(-4, 5, size=(3, d)).astype(np.float64)
    w_up = rng.integers(-2, 3, size=(f, d)).astype(np.float64)
    w_down = rng.integers(-2, 3, size=(5, f)).astype(np.float64)
    for k_in, k_mid in itertools.product((0, 4, 9), (0, 3, 7)):
        out = oracle.ffn_relu2(x, k_in, w_up, k_mid, w_down)
        for r in range(3):
            s1 = _topk_loop(list(x[r]), k_in)
            u = [sum(x[r, j] * w_up[i, j] for j in s1) for i in range(f)]
            h = [v * v if v > 0 else 0.0 for v in u]
            s2 = _topk_loop(h, k_mid)
            y = [sum(h[i] * w_down[o, i] for i in s2) for o in range(5)]
            assert out["u"][r].tolist() == u
            assert out["h"][r].tolist() == h
            assert set(np.nonzero(out["mask2"][r])[0].tolist()) == s2
            assert out["y"][r].tolist() == y
        down = oracle.ffn_relu2_down_from(out["h"], k_mid, w_down)
        assert np.array_equal(down["y"], out["y"])


def test_ffn_relu2_glu_brute_force():
    rng = np.random.default_rng(3)
    d, f = 9, 8
    x = rng.integers(-4, 5, size=(3, d)).astype(np.float64)
    wg = rng.integers(-2, 3, size=(f, d)).astype(np.float64)
    wu = rng.integers(-2, 3, size=(f, d)).astype(np.float64)
    wd = rng.integers(-2, 3, size=(5, f)).astype(np.float64)
    for k_in, k_mid in itertools.product((0, 4, 9), (0, 3, 8)):
        out = oracle.ffn_relu2_glu(x, k_in, wg, wu, k_mid, wd)
        for r in range(3):
            s1 = _topk_loop(list(x[r]), k_in)
            g = [sum(x[r, j] * wg[i, j] for j in s1) for i in range(f)]
            u = [sum(x[r, j] * wu[i, j] for j in s1) for i in range(f)]
            h = [(gv * gv if gv > 0 else 0.0) * uv for gv, uv in zip(g, u)]
            s2 = _topk_loop(h, k_mid)          # by |h|: h can be negative
            y = [sum(h[i] * wd[o, i] for i in s2) for o in range(5)]
            assert out["g"][r].tolist() == g and out["u"][r].tolist() == u
            assert out["h"][r].tolist() == h
            assert set(np.nonzero(out["mask2"][r])[0].tolist()) == s2
            assert out["y"][r].tolist() == y
        # the second half is the relu2 FFN's, started from this h
        down = oracle.ffn_relu2_down_from(out["h"], k_mid, wd)
        assert np.array_equal(down["y"], out["y"])
    # a negative intermediate can win the second selection by magnitude
    h = np.array([[4.0, -9.0, 1.0, 0.0]])
    m2, _, _, _ = oracle.topk_select(oracle.magnitude(h), 1)
    assert m2.tolist() == [[0, 1, 0, 0]]


def test_ffn_drelu_brute_force():
    rng = np.random.default_rng(4)
    d, f = 8, 10
    x = rng.integers(-3, 4, size=(2, d)).astype(np.float64)
    wg = rng.integers(-2, 3, size=(f, d)).astype(np.float64)
    wu = rng.integers(-2, 3, size=(f, d)).astype(np.float64)
    wd = rng.integers(-2, 3, size=(6, f)).astype(np.float64)
    bg = rng.integers(-2, 3, size=f).astype(np.float64)
    bu = rng.integers(-2, 3, size=f).astype(np.float64)
    out = oracle.ffn_drelu(x, wg, bg, wu, bu, wd)
    for r in range(2):
        g = [sum(x[r, j] * wg[i, j] for j in range(d)) + bg[i] for i in range(f)]
        u = [sum(x[r, j] * wu[i, j] for j in range(d)) + bu[i] for i in range(f)]
        h = [max(a, 0.0) * max(b, 0.0) for a, b in zip(g, u)]
        nz = [i for i in range(f) if h[i] != 0.0]
        y = [sum(h[i] * wd[o, i] for i in nz) for o in range(6)]
        assert out["g"][r].tolist() == g and out["u"][r].tolist() == u
        assert out["h"][r].tolist() == h
        assert out["nz_idx"][r].tolist() == nz and out["nz_count"][r] == len(nz)
        assert out["y"][r].tolist() == y
        assert np.all(out["T_g"][r] >= np.abs(out["g"][r]))
