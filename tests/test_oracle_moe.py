"""Pins of the oracle's MoE dReLU FFN: routing against closed forms and brute
force, one expert reducing to the (separately pinned) dReLU FFN, and the
two-expert output reducing to one dReLU FFN over the concatenated experts
with the routing weights folded into the down projection."""
import itertools
import math

import numpy as np
import pytest

import oracle


def _onehot_router(logits):
    """x = e_0 and W_router[:, 0] = logits gives exactly those logits."""
    e = len(logits)
    x = np.zeros((1, 4))
    x[0, 0] = 1.0
    wr = np.zeros((e, 4))
    wr[:, 0] = logits
    return x, wr


@pytest.mark.parametrize("logits,k,experts,weights", [
    ([0.0, 1.0, 3.0, 3.0], 2, [2, 3], [0.5, 0.5]),
    ([5.0, 1.0, 5.0, 0.0], 2, [0, 2], [0.5, 0.5]),
    ([2.0, 0.0, 1.0], 2, [0, 2], [1 / (1 + math.exp(-1)), math.exp(-1) / (1 + math.exp(-1))]),
    ([1.0, 1.0, 1.0], 1, [0], [1.0]),
    ([-1.0, -3.0, -2.0, -0.5], 3, [0, 2, 3], None),
])
def test_route_closed_forms(logits, k, experts, weights):
    x, wr = _onehot_router(logits)
    lg, ex, w, _ = oracle.moe_route(x, wr, k)
    assert np.array_equal(lg[0], logits)
    assert ex[0].tolist() == experts
    if weights is None:
        z = np.exp(np.array(logits)[experts])
        weights = z / z.sum()
    assert np.allclose(w[0], weights, rtol=1e-15, atol=0)
    assert math.isclose(w[0].sum(), 1.0, rel_tol=1e-15)


def test_route_brute_force():
    rng = np.random.default_rng(2)
    for _ in range(40):
        e, k = int(rng.integers(2, 7)), 0
        k = int(rng.integers(1, e + 1))
        logits = rng.integers(-2, 3, size=e).astype(np.float64)   # ties
        x, wr = _onehot_router(logits)
        _, ex, _, _ = oracle.moe_route(x, wr, k)
        ok = [set(s) for s in itertools.combinations(range(e), k)
              if all(logits[i] > logits[j] or (logits[i] == logits[j] and i < j)
                     for i in s for j in range(e) if j not in s)]
        assert len(ok) == 1 and set(ex[0].tolist()) == ok[0]


def _experts(rng, e, d, ffn, bias):
    wg = rng.normal(0, 0.3, size=(e, ffn, d))
    wu = rng.normal(0, 0.3, size=(e, ffn, d))
    wd = rng.normal(0, 0.3, size=(e, d, ffn))
    bg = np.full((e, ffn), bias)
    bu = np.full((e, ffn), bias)
    return wg, bg, wu, bu, wd


def test_single_expert_is_the_drelu_ffn():
    rng = np.random.default_rng(4)
    d, ffn = 6, 10
    x = rng.normal(size=(3, d))
    wr = rng.normal(size=(1, d))
    wg, bg, wu, bu, wd = _experts(rng, 1, d, ffn, -0.2)
    out = oracle.moe_drelu_ffn(x, wr, 1, wg, bg, wu, bu, wd)
    assert np.all(out["weights"] == 1.0)
    for r in range(3):
        ref = oracle.ffn_drelu(x[r:r + 1], wg[0], bg[0], wu[0], bu[0], wd[0])
        assert np.array_equal(out["y"][r], ref["y"][0])
        assert np.array_equal(out["h"][r, 0], ref["h"][0])


def test_two_experts_fold_into_one_concatenated_ffn():
    rng = np.random.default_rng(5)
    d, ffn, e = 8, 12, 5
    x = rng.normal(size=(4, d))
    wr = rng.normal(size=(e, d))
    wg, bg, wu, bu, wd = _experts(rng, e, d, ffn, -0.3)
    out = oracle.moe_drelu_ffn(x, wr, 2, wg, bg, wu, bu, wd)
    for r in range(4):
        e1, e2 = out["experts"][r]
        w1, w2 = out["weights"][r]
        cat = oracle.ffn_drelu(x[r:r + 1], np.vstack([wg[e1], wg[e2]]), np.concatenate([bg[e1], bg[e2]]),
                               np.vstack([wu[e1], wu[e2]]), np.concatenate([bu[e1], bu[e2]]),
                               np.hstack([w1 * wd[e1], w2 * wd[e2]]))
        assert np.allclose(out["y"][r], cat["y"][0], rtol=1e-12, atol=1e-12)
        assert np.allclose(out["h"][r].ravel(), cat["h"][0], rtol=0, atol=0)
    assert np.all(np.abs(out["y"]) <= out["T_y"] * (1 + 1e-12))
