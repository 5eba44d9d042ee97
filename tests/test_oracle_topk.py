"""Pins of the oracle's top-K selection against what the pages fix.

The pages (Q-Sparse news article, "Sparsification with the Top-K function")
define the mask as 1 at the K entries of largest |x| and 0 elsewhere; the
lower-index tie-break is the reading taken.  The pins: hand-worked examples,
brute force over every K-subset of tiny rows, an independent pure-Python
sort, special cases and the mask invariants.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dominates(mag, i, j):
    """True iff entry i ranks strictly before entry j (magnitude, then index)."""
    return mag[i] > mag[j] or (mag[i] == mag[j] and i < j)


def test_worked_examples():
    with open(os.path.join(GOLDEN, "topk_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.array([c["x"]], dtype=np.float64)
        mask, idx, tau, cut = oracle.topk_select(oracle.magnitude(x), c["k"])
        assert idx[0].tolist() == c["idx"], c["why"]
        assert mask[0].tolist() == c["mask"], c["why"]
        want_tau = float("inf") if c["tau"] == "inf" else c["tau"]
        assert tau[0] == want_tau and cut[0] == c["cutoff"], c["why"]


@pytest.mark.parametrize("d", [1, 2, 5, 7, 9])
def test_brute_force_subsets(d):
    rng = np.random.default_rng(d)
    for trial in range(12):
        # few distinct magnitudes and both signs, so ties are everywhere
        x = rng.integers(-3, 4, size=d).astype(np.float64)
        if trial % 3 == 0:
            x = rng.standard_normal(d)
        mag = np.abs(x)
        for k in range(d + 1):
            good = []
            for sub in itertools.combinations(range(d), k):
                s = set(sub)
                if all(_dominates(mag, i, j) for i in s for j in range(d) if j not in s):
                    good.append(sub)
            assert len(good) == 1, "the tie-break must make the selected set unique"
            mask, idx, _, _ = oracle.topk_select(mag[None, :], k)
            assert tuple(idx[0].tolist()) == good[0]
            assert sorted(np.nonzero(mask[0])[0].tolist()) == list(good[0])


def test_independent_python_sort():
    rng = np.random.default_rng(7)
    x = rng.integers(-20, 21, size=(6, 300)).astype(np.float64) * 0.5
    x[2] = 0.0
    x[3, ::2] = -x[3, 1::2]
    mag = np.abs(x)
    for k in (0, 1, 37, 150, 299, 300):
        mask, idx, tau, cut = oracle.topk_select(mag, k)
        for r in range(x.shape[0]):
            order = sorted(range(300), key=lambda j: (-mag[r, j], j))
            assert idx[r].tolist() == sorted(order[:k])
            if k:
                assert tau[r] == mag[r, order[k - 1]]


def test_descriptor_reproduces_mask_and_invariants():
    rng = np.random.default_rng(11)
    x = np.round(rng.standard_t(4, size=(5, 257)), 1)      # many ties
    mag = oracle.magnitude(x)
    for k in (0, 1, 100, 256, 257):
        mask, idx, tau, cut = oracle.topk_select(mag, k)
        assert (mask.sum(axis=1) == k).all()
        j = np.arange(257)
        for r in range(5):
            assert np.all(np.diff(idx[r]) > 0)
            assert np.array_equal(np.nonzero(mask[r])[0], idx[r])
            rule = (mag[r] > tau[r]) | ((mag[r] == tau[r]) & (j < cut[r]))
            assert np.array_equal(rule.astype(np.uint8), mask[r])
            if k:
                sel_min = mag[r][mask[r] == 1].min()
                unsel = mag[r][mask[r] == 0]
                assert unsel.size == 0 or sel_min >= unsel.max()


def test_special_cases():
    x = np.full((2, 10), -1.5)
    mask, idx, tau, cut = oracle.topk_select(oracle.magnitude(x), 4)
    assert (idx == np.arange(4)).all() and (cut == 4).all() and (tau == 1.5).all()
    z = np.zeros((1, 6))
    z[0, 3] = -0.0
    mask, idx, tau, cut = oracle.topk_select(oracle.magnitude(z), 2)
    assert idx[0].tolist() == [0, 1]
    with pytest.raises(ValueError):
        oracle.topk_select(np.zeros((1, 3)), 4)
