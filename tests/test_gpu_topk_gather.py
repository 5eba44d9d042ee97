"""GPU parity of qs_topk_gather_linear_acc: Y += (X (.) M) . W^T with M the
per-row top-k mask of the fp32 X by |x| (ties to the lower index), found by
every workgroup of the gather itself (Q-Sparse news article, Top-K section;
Turbo Sparse summary, Eq. 3-4 for the same selection on the FFN
intermediate).

Bound: fp32 products and sums, |y - (y0 + y_ref)| <= 1e-5 * (T + |y0|) with
T = sum over the oracle's selected j of |x_j w_j|.  One entry selected
wrongly moves y by about T / k, far outside that bound, so the bound also
checks the selection.
"""
import numpy as np
import pytest

import datagen
import oracle
from gpu_util import note, to_dev

pytestmark = pytest.mark.gpu

EPS = 1e-5


def _rows(kind, rng, rows, d):
    x = datagen.student_t(rng, (rows, d)).astype(np.float32)
    if kind == "relu2":        # half zeros, as the FFN intermediate
        x = np.where(x > 0, x * x, 0.0).astype(np.float32)
    elif kind == "ties":       # long runs of equal magnitudes, both signs
        x = (np.round(x * 4) / 4).astype(np.float32)
    return x


def _check(qs, x, k, w):
    import torch
    rng = np.random.default_rng(x.shape[1] + k)
    y0 = rng.standard_normal((x.shape[0], w.shape[0])).astype(np.float32)
    y = to_dev(y0)
    qs.qs_topk_gather_linear_acc(to_dev(x), k, to_dev(np.ascontiguousarray(w.T), torch.bfloat16), y)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    mask, _, _, _ = oracle.topk_select(oracle.magnitude(x), k)
    ref, t = oracle.sparse_linear(x, w, mask)
    bound = EPS * (t + np.abs(y0))
    err = np.abs(got - (y0.astype(np.float64) + ref))
    assert np.all(err <= bound), f"worst excess {np.max(err - bound)} at {np.unravel_index(np.argmax(err - bound), err.shape)}"


@pytest.mark.parametrize("kind", ["plain", "relu2", "ties"])
@pytest.mark.parametrize("rows,d,n", [(1, 96, 8), (1, 1000, 520), (3, 4104, 264),
                                      (1, 11008, 4096), (2, 16384, 520)])
def test_topk_gather_acc(gpu_lib, kind, rows, d, n):
    rng = np.random.default_rng(d * 3 + n + rows + len(kind))
    x = _rows(kind, rng, rows, d)
    w = datagen.bf16_round(datagen.normal(rng, (n, d), 0.02))
    nnz = int(np.count_nonzero(x[0]))
    for k in sorted({0, 1, (2 * d) // 5, min(d, nnz + 3), d - 1, d}):
        note(f"topk-gather acc {kind} rows={rows} d={d} n={n} k={k}")
        _check(gpu_lib, x, k, w)
