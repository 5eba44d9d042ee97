"""Pins of the oracle's Block Q-Sparse selection (N:M top-K per contiguous
block of features): brute force over every subset of each block, reduction to
the per-row top-K oracle applied to each block alone, special cases."""
import itertools

import numpy as np
import pytest

import oracle


def _brute_block(mag_block, n_keep):
    """The unique n_keep-subset S with: every member beats (magnitude higher,
    or equal with a lower index) every non-member."""
    m = len(mag_block)
    found = []
    for s in itertools.combinations(range(m), n_keep):
        out = [j for j in range(m) if j not in s]
        ok = all(mag_block[i] > mag_block[j] or (mag_block[i] == mag_block[j] and i < j)
                 for i in s for j in out)
        if ok:
            found.append(set(s))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("n_keep,block", [(2, 4), (1, 4), (3, 4), (2, 8), (4, 4), (0, 4)])
def test_block_select_brute_force(n_keep, block):
    rng = np.random.default_rng(n_keep * 10 + block)
    # small integer magnitudes: many ties inside blocks
    mag = rng.integers(0, 4, size=(5, 6 * block)).astype(np.float64)
    mask = oracle.block_topk_select(mag, n_keep, block)
    for r in range(mag.shape[0]):
        for b0 in range(0, mag.shape[1], block):
            sel = set(np.nonzero(mask[r, b0:b0 + block])[0].tolist())
            assert sel == _brute_block(mag[r, b0:b0 + block].tolist(), n_keep)
    assert np.all(mask.reshape(5, -1, block).sum(axis=2) == n_keep)


def test_block_select_is_rowwise_topk_of_each_block():
    rng = np.random.default_rng(3)
    x = rng.standard_t(4, size=(7, 64)).astype(np.float32)
    x[0, :8] = 1.5                      # ties
    x[1, 4:8] = [-2.0, 2.0, -2.0, 0.0]  # x next to -x
    mag = oracle.magnitude(x)
    mask = oracle.block_topk_select(mag, 2, 4)
    for b0 in range(0, 64, 4):
        m_b, _, _, _ = oracle.topk_select(mag[:, b0:b0 + 4], 2)
        assert np.array_equal(mask[:, b0:b0 + 4], m_b)


def test_block_select_special_cases():
    const = np.full((2, 8), 3.0)
    assert oracle.block_topk_select(const, 2, 4).tolist() == [[1, 1, 0, 0, 1, 1, 0, 0]] * 2
    zeros = np.zeros((1, 4))
    assert oracle.block_topk_select(zeros, 2, 4).tolist() == [[1, 1, 0, 0]]
    desc = np.array([[1.0, 2.0, 3.0, 4.0]])
    assert oracle.block_topk_select(desc, 2, 4).tolist() == [[0, 0, 1, 1]]
    with pytest.raises(ValueError):
        oracle.block_topk_select(np.zeros((1, 6)), 2, 4)
