"""Pins of the CPU oracle's backward (straight-through estimator) against the
forward oracle, which the other oracle tests pin on their own.

L(X, W) = sum(dY (.) Y) with Y = (X (.) M) . W^T is linear in W for a fixed
mask and linear in X wherever the mask does not change, so an exact finite
difference of the forward (integer-valued data and power-of-two steps keep
every float64 sum exact) gives each gradient entry independently of the
backward formulas.
"""
import numpy as np
import pytest

import oracle


def _loss(x, w, mask, gy):
    y, _ = oracle.sparse_linear(x, w, mask)
    return float(np.sum(np.asarray(gy, dtype=np.float64) * y))


def _int_case(seed, r, d, n, k):
    rng = np.random.default_rng(seed)
    # distinct magnitudes in every row, so the top-K set is stable under tiny steps
    x = np.stack([rng.permutation(np.arange(1, d + 1)) * rng.choice([-1, 1], d) for _ in range(r)]).astype(np.float64)
    w = rng.integers(-3, 4, size=(n, d)).astype(np.float64)
    gy = rng.integers(-4, 5, size=(r, n)).astype(np.float64)
    mask, _, _, _ = oracle.topk_select(oracle.magnitude(x), k)
    return x, w, gy, mask


@pytest.mark.parametrize("r,d,n,k", [(3, 7, 5, 3), (2, 9, 4, 0), (4, 6, 3, 6), (1, 5, 8, 2)])
def test_dw_is_exact_finite_difference_of_forward(r, d, n, k):
    x, w, gy, mask = _int_case(10 + r, r, d, n, k)
    out = oracle.sparse_linear_backward(x, w, mask, gy)
    assert out["dw"].shape == (n, d)
    l0 = _loss(x, w, mask, gy)
    for o in range(n):
        for j in range(d):
            w1 = w.copy()
            w1[o, j] += 1.0
            assert _loss(x, w1, mask, gy) - l0 == out["dw"][o, j]


@pytest.mark.parametrize("r,d,n,k", [(3, 7, 5, 3), (2, 9, 4, 4), (1, 5, 8, 5)])
def test_dx_is_ste_copy_of_the_selected_gradient(r, d, n, k):
    x, w, gy, mask = _int_case(20 + r, r, d, n, k)
    out = oracle.sparse_linear_backward(x, w, mask, gy)
    assert out["dx"].shape == (r, d)
    step = 2.0 ** -20            # far below the gap between distinct magnitudes
    l0 = _loss(x, w, mask, gy)
    ones = np.ones_like(mask)
    l0_dense = _loss(x, w, ones, gy)
    for i in range(r):
        for j in range(d):
            x1 = x.copy()
            x1[i, j] += step
            m1, _, _, _ = oracle.topk_select(oracle.magnitude(x1), k)
            assert np.array_equal(m1, mask)            # the step leaves the selection alone
            true_g = (_loss(x1, w, m1, gy) - l0) / step
            if mask[i, j]:
                # selected entries: the STE value is the true gradient
                assert out["dx"][i, j] == true_g
            else:
                # masked-out entries: the true gradient is zero, the STE passes
                # the gradient of the sparsified tensor through anyway
                assert true_g == 0.0
            # everywhere: the gradient the dense product would have
            assert out["dx"][i, j] == (_loss(x1, w, ones, gy) - l0_dense) / step


def test_dx_not_masked_and_dw_columns_outside_union_are_zero():
    x, w, gy, mask = _int_case(7, 3, 10, 6, 2)
    out = oracle.sparse_linear_backward(x, w, mask, gy)
    unsel = mask == 0
    assert np.any(out["dx"][unsel] != 0.0)            # STE: not masked
    union = mask.any(axis=0)
    assert np.all(out["dw"][:, ~union] == 0.0)
    assert np.any(out["dw"][:, union] != 0.0)


def test_full_k_reduces_to_dense_linear_gradients():
    x, w, gy, _ = _int_case(8, 4, 6, 5, 6)
    ones = np.ones((4, 6), dtype=np.uint8)
    out = oracle.sparse_linear_backward(x, w, ones, gy)
    # textbook gradients of Y = X W^T written as explicit loops
    dx = np.zeros((4, 6))
    dw = np.zeros((5, 6))
    for r in range(4):
        for o in range(5):
            for j in range(6):
                dx[r, j] += gy[r, o] * w[o, j]
                dw[o, j] += gy[r, o] * x[r, j]
    assert np.array_equal(out["dx"], dx) and np.array_equal(out["dw"], dw)


def test_error_scales_bound_the_gradients():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 12))
    w = rng.standard_normal((7, 12))
    gy = rng.standard_normal((5, 7))
    mask, _, _, _ = oracle.topk_select(oracle.magnitude(x), 4)
    out = oracle.sparse_linear_backward(x, w, mask, gy)
    assert np.all(np.abs(out["dx"]) <= out["T_dx"] * (1 + 1e-12))
    assert np.all(np.abs(out["dw"]) <= out["T_dw"] * (1 + 1e-12))
    assert np.all(out["T_dw"][:, ~mask.astype(bool).any(axis=0)] == 0.0)
