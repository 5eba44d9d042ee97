"""GPU parity of the small-batch squared-ReLU FFN called without the index
list and count of the intermediate: its selection of h writes only the top-k
descriptor (tau, cutoff), which the down gather applies to h.

Q-Sparse's top-k on the intermediate: Turbo Sparse summary, Eq. 3-4 (the
top-k% of h by |h| before W_down); ties go to the lower index.

With one token the down gather's workgroups find the descriptor themselves
(no descriptor launch).  Each case runs the bare call in both reduction
modes beside the call with every optional output on, whose index list of h
comes from the selection launch and is checked against the oracle's
selection of the same h index by index, and:

* y of the bare call is within the fp32 summation bound (1e-5 * T_y) of the
  oracle's down projection of the call's own h (h has no atomics, so it is
  the same in every call) over the oracle's selection: one intermediate
  entry selected wrongly moves y by about T_y / k_mid, far more;
* with several tokens (the same gather kernel in both calls), fixed-order
  sums: y of the bare call is bitwise equal to y of the full call.

The inputs steer the selection into each branch of its search:
plain rows, rows whose boundary falls among many equal values (the long-list
and tie branches), rows with fewer nonzero entries than k (the boundary
among zeros), rows of a few distinct values (a boundary bin taken whole),
and the trivial k.
"""
import numpy as np
import pytest

import datagen
import oracle
from gpu_util import assert_within, note, reduction_mode, to_dev

pytestmark = pytest.mark.gpu

TOL_BF16 = 4e-3
SUM_EPS = 1e-5    # the fp32 tolerance: bound of the gathers' fp32 summation


def _weights(kind, rng, d, f):
    """W_up [f, d] (oracle layout) that makes h = relu(x . W_up^T)^2 of the
    given kind; W_down [d, f]."""
    w_up = datagen.normal(rng, (f, d), 0.02)
    if kind == "ties":
        # a block of 600 identical rows (three quarters of them when f <
        # 800): that many equal values of h among the others
        n = min(600, (3 * f) // 4)
        w_up[:n] = w_up[0]
        perm = rng.permutation(f)
        w_up = w_up[perm]
    elif kind == "ties_small":
        # 100 equal values: a short list whose boundary bin has > 64 keys
        n = min(100, f // 2)
        w_up[:n] = w_up[0]
        w_up = w_up[rng.permutation(f)]
    elif kind == "few_values":
        # three distinct rows repeated: h takes three values (and zeros)
        base = w_up[:3].copy()
        w_up = base[rng.integers(0, 3, size=f)]
    w_down = datagen.normal(rng, (d, f), 0.02)
    return datagen.bf16_round(w_up), datagen.bf16_round(w_down)


def _run(qs, x, k_in, k_mid, wu, wd):
    import torch
    xd = to_dev(x, torch.bfloat16)
    wud = to_dev(np.ascontiguousarray(wu.T), torch.bfloat16)
    wdd = to_dev(np.ascontiguousarray(wd.T), torch.bfloat16)
    y_bare = torch.empty((x.shape[0], wd.shape[0]), dtype=torch.float32, device=xd.device)
    qs.qs_sparse_ffn(xd, qs.ACT_RELU2, k_in, k_mid, wud, wdd, y=y_bare)
    y_full, h, idx, cnt = qs.qs_sparse_ffn(xd, qs.ACT_RELU2, k_in, k_mid, wud, wdd,
                                          want_h=True, want_mid=True)
    torch.cuda.synchronize()
    return y_bare.cpu().numpy(), y_full.cpu().numpy(), h.cpu().numpy(), idx.cpu().numpy()


def _check(qs, x, k_in, k_mid, wu, wd, what):
    hvals = None
    for det in (True, False):
        note(f"descriptor select {what} det={det} rows={x.shape[0]} d={x.shape[1]} "
             f"ffn={wu.shape[0]} k_mid={k_mid}")
        with reduction_mode(qs, det):
            y_bare, y_full, h, idx = _run(qs, x, k_in, k_mid, wu, wd)
        if det and x.shape[0] > 1:
            assert np.array_equal(y_bare.view(np.uint32), y_full.view(np.uint32)), \
                f"{what}: bare call (descriptor only) differs from the full call"
        down = oracle.ffn_relu2_down_from(h, k_mid, wd)
        for r in range(x.shape[0]):
            assert np.array_equal(idx[r, :k_mid], down["idx2"][r]), f"{what}: index list row {r}"
        assert_within(y_bare, down["y"], down["T_y"], SUM_EPS, f"{what} y")
        hvals = h
    return hvals


@pytest.mark.parametrize("rows", [1, 3])
@pytest.mark.parametrize("f", [96, 520, 1000, 4104, 11008, 16384])
@pytest.mark.parametrize("kind", ["plain", "ties", "ties_small", "few_values"])
def test_desc_select_kinds(gpu_lib, rows, f, kind):
    d = 256
    rng = np.random.default_rng(f * 7 + len(kind) + 1000 * rows)
    x = datagen.bf16_round(datagen.student_t(rng, (rows, d)))
    wu, wd = _weights(kind, rng, d, f)
    k_in = (2 * d) // 5
    h = None
    for frac in (0.4, 0.05, 0.3):
        k_mid = max(1, int(frac * f))
        h = _check(gpu_lib, x, k_in, k_mid, wu, wd, f"{kind} k_mid={k_mid}")
    if kind in ("ties", "ties_small", "few_values"):
        # a boundary inside the block of equal values of row 0, whatever its rank
        mag = np.abs(h[0].astype(np.float64))
        if not np.any(mag > 0):
            return
        vals, counts = np.unique(mag[mag > 0], return_counts=True)
        v = vals[np.argmax(counts)]
        above = int(np.sum(mag > v))
        k_mid = above + int(counts.max()) // 2
        if 0 < k_mid < f:
            _check(gpu_lib, x, k_in, k_mid, wu, wd, f"{kind} boundary in the ties k_mid={k_mid}")
        # the block taken whole
        k_mid = above + int(counts.max())
        if 0 < k_mid < f:
            _check(gpu_lib, x, k_in, k_mid, wu, wd, f"{kind} ties taken whole k_mid={k_mid}")


@pytest.mark.parametrize("f", [520, 11008])
def test_desc_select_edges(gpu_lib, f):
    """k past the nonzero count (the boundary among zeros), k = nnz, k = 0,
    1 and f."""
    d = 256
    rng = np.random.default_rng(f + 3)
    x = datagen.bf16_round(datagen.student_t(rng, (1, d)))
    wu, wd = _weights("plain", rng, d, f)
    _, _, h, _ = _run(gpu_lib, x, (2 * d) // 5, 1, wu, wd)
    nnz = int(np.count_nonzero(h))
    assert 0 < nnz < f
    for k_mid in sorted({0, 1, nnz - 1, nnz, nnz + 1, (nnz + f) // 2, f - 1, f}):
        _check(gpu_lib, x, (2 * d) // 5, k_mid, wu, wd, f"edge k_mid={k_mid} nnz={nnz}")
