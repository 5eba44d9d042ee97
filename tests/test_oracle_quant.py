"""Pins of the oracle's quantised path.

The quantiser formulas are missing from the pages; the readings (absmax-127
activations with eps in the denominator, ternary weights with alpha = mean
|W|) are pinned here by exact rational arithmetic, special rows, symmetry
and integer brute force.  Parity to the paper's own formulas is unpinned.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact import fl32, rint_even, ulp32

EPS32 = Fraction(float(np.float32(1e-5)))


def test_quant_matches_exact_binary32_chain():
    rng = np.random.default_rng(21)
    x = rng.standard_t(4, size=(6, 40)).astype(np.float32)
    x[1] *= 1e-6
    x[2, 5] = 0.0
    q, s, gamma = oracle.absmax_quant_i8(x)
    for r in range(x.shape[0]):
        g = max(abs(Fraction(float(v))) for v in x[r])
        assert Fraction(float(gamma[r])) == g
        den = fl32(g + EPS32)
        s_exact = fl32(Fraction(127) / den)
        assert Fraction(float(s[r])) == s_exact
        for j in range(x.shape[1]):
            want = rint_even(fl32(Fraction(float(x[r, j])) * s_exact))
            want = min(127, max(-128, want))
            assert int(q[r, j]) == want


def test_quant_special_rows():
    x = np.zeros((4, 8), dtype=np.float32)
    x[0, 3] = -2.5                  # one-hot
    x[1, :] = 0.75                  # constant
    x[3, :] = np.linspace(-1, 1, 8, dtype=np.float32)
    q, s, _ = oracle.absmax_quant_i8(x)
    assert q[0].tolist() == [0, 0, 0, -127, 0, 0, 0, 0]
    assert (q[1] == 127).all()
    assert (q[2] == 0).all() and np.isfinite(s[2]) and s[2] > 0     # eps guards the zero row
    assert q[3, 0] == -127 and q[3, -1] == 127
    assert (np.abs(q) <= 127).all()
    qn, sn, _ = oracle.absmax_quant_i8(-x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)


def test_quant_then_topk_constant_row_takes_first_k():
    x = np.full((1, 20), -3.0, dtype=np.float32)
    q, _, _ = oracle.absmax_quant_i8(x)
    _, idx, _, _ = oracle.topk_select(oracle.magnitude(q), 7)
    assert idx[0].tolist() == list(range(7))


def test_ternarize_alpha_and_codes():
    w = np.array([[0.5, -1.0, 0.25, 0.0], [2.0, -0.125, 0.75, -0.5]], dtype=np.float32)
    t, alpha = oracle.ternarize(w)
    exact_mean = sum(abs(Fraction(float(v))) for v in w.ravel()) / w.size     # 5.125 / 8
    assert Fraction(float(alpha)) == exact_mean
    # |w| / (alpha+eps): 0.78 -> 1, 1.56 -> 1, 0.39 -> 0, 0, 3.12 -> 1, 0.195 -> 0, 1.17 -> 1, 0.78 -> 1
    assert t.tolist() == [[1, -1, 0, 0], [1, 0, 1, -1]]


def test_ternarize_random_against_thresholds():
    rng = np.random.default_rng(23)
    w = rng.normal(0, 0.02, size=(33, 64)).astype(np.float32)
    t, alpha = oracle.ternarize(w)
    exact_mean = sum(abs(Fraction(float(v))) for v in w.ravel()) / w.size
    assert abs(Fraction(float(alpha)) - exact_mean) <= ulp32(exact_mean)
    assert set(np.unique(t).tolist()) <= {-1, 0, 1}
    den = fl32(Fraction(float(alpha)) + EPS32)
    for v, tv in zip(w.ravel(), t.ravel()):
        want = max(-1, min(1, rint_even(fl32(Fraction(float(v)) / den))))
        assert int(tv) == want


def test_unpack_ternary_layout():
    # feature row 0: columns 0..3 = (0, +1, 0, -1) -> codes 00 01 00 11 -> 0b11000100
    # feature row 1: columns 0..3 = (-1, -1, +1, 0) -> codes 11 11 01 00 -> 0b00011111
    packed = np.array([[0b11000100], [0b00011111]], dtype=np.uint8)
    t = oracle.unpack_ternary(packed, 4)
    assert t.tolist() == [[0, -1], [1, -1], [0, 1], [-1, 0]]
    with pytest.raises(ValueError):
        oracle.unpack_ternary(np.array([[0b10]], dtype=np.uint8), 4)


def test_i8t_linear_brute_force():
    rng = np.random.default_rng(29)
    x = rng.standard_t(4, size=(3, 24)).astype(np.float32)
    w = rng.normal(0, 0.02, size=(5, 24)).astype(np.float32)
    q, s, _ = oracle.absmax_quant_i8(x)
    t, alpha = oracle.ternarize(w)
    mask, _, _, _ = oracle.topk_select(oracle.magnitude(q), 9)
    acc, y = oracle.i8t_linear(q, s, t, alpha, mask)
    for r in range(3):
        scale = fl32(Fraction(float(alpha)) / Fraction(float(s[r])))
        for o in range(5):
            a = sum(int(q[r, j]) * int(t[o, j]) for j in range(24) if mask[r, j])
            assert acc[r, o] == a
            assert Fraction(float(y[r, o])) == fl32(Fraction(a) * scale)


def test_i8t_zero_row_gives_zero():
    x = np.zeros((1, 16), dtype=np.float32)
    q, s, _ = oracle.absmax_quant_i8(x)
    t = np.ones((3, 16), dtype=np.int8)
    mask, _, _, _ = oracle.topk_select(oracle.magnitude(q), 5)
    acc, y = oracle.i8t_linear(q, s, t, np.float32(0.02), mask)
    assert (acc == 0).all() and (y == 0).all()
