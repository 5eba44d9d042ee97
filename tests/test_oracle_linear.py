"""Pins of the oracle's sparse-activation linear Y = (X (.) M) . W^T.

Pins: hand-worked examples, exact rational triple loops, K = D reducing to
the dense product (computed here by the triple loop, not by the oracle's
matmul), linearity over complementary masks, and non-square shapes so a
transposed operand cannot pass.
"""
import json
import os
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _loop_product(x, w, mask):
    rows, d = x.shape
    n = w.shape[0]
    y = [[Fraction(0)] * n for _ in range(rows)]
    t = [[Fraction(0)] * n for _ in range(rows)]
    for r in range(rows):
        for o in range(n):
            for j in range(d):
                if mask[r, j]:
                    p = Fraction(float(x[r, j])) * Fraction(float(w[o, j]))
                    y[r][o] += p
                    t[r][o] += abs(p)
    return y, t


def test_worked_examples():
    with open(os.path.join(GOLDEN, "linear_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.array(c["x"])
        w = np.array(c["w"])
        mask, _, _, _ = oracle.topk_select(oracle.magnitude(x), c["k"])
        y, t = oracle.sparse_linear(x, w, mask)
        assert y.tolist() == c["y"], c["why"]
        assert t.tolist() == c["T"], c["why"]


def test_against_exact_loops():
    rng = np.random.default_rng(3)
    for (rows, d, n, k) in [(1, 7, 3, 3), (3, 11, 5, 4), (2, 16, 9, 16), (4, 13, 2, 0)]:
        x = rng.standard_t(4, size=(rows, d)).astype(np.float32)
        w = rng.normal(0, 0.02, size=(n, d)).astype(np.float32)
        mask, _, _, _ = oracle.topk_select(oracle.magnitude(x), k)
        y, t = oracle.sparse_linear(x, w, mask)
        ye, te = _loop_product(x, w, mask)
        for r in range(rows):
            for o in range(n):
                scale = float(te[r][o])
                assert abs(Fraction(y[r, o]) - ye[r][o]) <= Fraction(1e-13) * (scale + 1e-300)
                assert abs(Fraction(t[r, o]) - te[r][o]) <= Fraction(1e-13) * (scale + 1e-300)


def test_integer_valued_is_exact():
    rng = np.random.default_rng(5)
    x = rng.integers(-9, 10, size=(3, 24)).astype(np.float64)
    w = rng.integers(-2, 3, size=(10, 24)).astype(np.float64)
    mask, _, _, _ = oracle.topk_select(oracle.magnitude(x), 10)
    y, _ = oracle.sparse_linear(x, w, mask)
    ye, _ = _loop_product(x, w, mask)
    assert [[Fraction(v) for v in row] for row in y.tolist()] == ye


def test_k_equal_d_is_the_dense_product():
    rng = np.random.default_rng(9)
    x = rng.integers(-5, 6, size=(2, 12)).astype(np.float64)
    w = rng.integers(-3, 4, size=(7, 12)).astype(np.float64)
    mask, _, _, _ = oracle.topk_select(oracle.magnitude(x), 12)
    y, _ = oracle.sparse_linear(x, w, mask)
    dense = [[sum(x[r, j] * w[o, j] for j in range(12)) for o in range(7)] for r in range(2)]
    assert y.tolist() == dense


def test_linearity_over_complementary_masks():
    rng = np.random.default_rng(13)
    x = rng.integers(-8, 9, size=(4, 30)).astype(np.float64)
    w = rng.integers(-4, 5, size=(6, 30)).astype(np.float64)
    mask, _, _, _ = oracle.topk_select(oracle.magnitude(x), 11)
    y1, _ = oracle.sparse_linear(x, w, mask)
    y2, _ = oracle.sparse_linear(x, w, 1 - mask)
    yall, _ = oracle.sparse_linear(x, w, np.ones_like(mask))
    assert np.array_equal(y1 + y2, yall)


def test_ste_is_identity():
    g = np.array([[1.5, -0.0, 0.0, -2.25, 7.0]], dtype=np.float32)
    out = oracle.ste_backward(g)
    assert out.dtype == g.dtype and np.array_equal(out.view(np.uint32), g.view(np.uint32))
    assert out is not g
