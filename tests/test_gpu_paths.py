"""Forced-path invariance: the same token through every internal path of an
entry point gives bitwise the same result.

The library picks a kernel by batch size and layout: the one-token column
kernel, the gathers with 2..8 token tiles, the 16-token matrix-core gathers,
the masked dense MFMA GEMM (QS_LAYOUT_W), the fixed-order and the atomic
split sums.  Each test places one token alone and inside batches that take
the other paths, with integer-valued inputs small enough that every product
and partial sum is exact in fp32, so every path must return the same bits;
integer-valued intermediates also put many equal magnitudes at every top-k
boundary, so the paths must agree on the tie rule too (Q-Sparse news
article, Top-K section; ties to the lower index).  The ternary path is exact
by construction (int32 sums).
"""
import numpy as np
import pytest

import datagen
from gpu_util import note, reduction_mode, to_dev

pytestmark = pytest.mark.gpu


def _ints(rng, shape, lo, hi):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def _batch_with(row, others, pos):
    b = others.copy()
    b[pos] = row
    return b


def test_paths_linear(gpu_lib):
    """One bf16 token: column kernel (alone), gather (3 tokens), matrix-core
    gather (16 tokens), masked dense MFMA (QS_LAYOUT_W, 40 tokens), in both
    reduction modes: y of that token bitwise equal everywhere."""
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    rng = np.random.default_rng(3)
    d, n, k = 1000, 520, 400
    w = _ints(rng, (n, d), -1, 1)
    tok = _ints(rng, (1, d), -6, 6)
    wt_dev, w_dev = to_dev(np.ascontiguousarray(w.T), bf), to_dev(w, bf)
    outs = {}
    for det in (False, True):
        with reduction_mode(qs, det):
            for rows, pos, lay in ((1, 0, qs.LAYOUT_WT), (3, 1, qs.LAYOUT_WT), (16, 9, qs.LAYOUT_WT),
                                   (40, 37, qs.LAYOUT_W)):
                x = _batch_with(tok[0], _ints(rng, (rows, d), -6, 6), pos)
                note(f"paths linear rows={rows} layout={lay} det={det}")
                y = qs.qs_sparse_linear(to_dev(x, bf), k, wt_dev if lay == qs.LAYOUT_WT else w_dev,
                                        layout=lay)
                torch.cuda.synchronize()
                outs[(rows, lay, det)] = y[pos].cpu().numpy()
    ref = outs[(1, qs.LAYOUT_WT, True)]
    for key, v in outs.items():
        assert np.array_equal(v.view(np.uint32), ref.view(np.uint32)), f"path {key} differs"


def test_paths_topk_gather_acc_vs_linear(gpu_lib):
    """fp32 token: the selection-in-gather accumulate call (alone and in a
    3-row call) against qs_sparse_linear's selection launch and gather."""
    import torch
    qs = gpu_lib
    rng = np.random.default_rng(4)
    d, n, k = 2048, 264, 819
    w = to_dev(np.ascontiguousarray(_ints(rng, (n, d), -1, 1).T), torch.bfloat16)
    tok = _ints(rng, (1, d), -9, 9)
    note("paths topk-gather acc vs linear")
    y_lin = qs.qs_sparse_linear(to_dev(tok), k, w)
    y1 = torch.zeros((1, n), dtype=torch.float32, device="cuda")
    qs.qs_topk_gather_linear_acc(to_dev(tok), k, w, y1)
    x3 = _batch_with(tok[0], _ints(rng, (3, d), -9, 9), 2)
    y3 = torch.zeros((3, n), dtype=torch.float32, device="cuda")
    qs.qs_topk_gather_linear_acc(to_dev(x3), k, w, y3)
    torch.cuda.synchronize()
    a, b, c = (t.cpu().numpy() for t in (y_lin[0], y1[0], y3[2]))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))


@pytest.mark.parametrize("act", ["relu2", "glu"])
def test_paths_ffn(gpu_lib, act):
    """One token of a squared-ReLU FFN: alone (selection inside both
    projections), in 3 tokens (selection launch, column kernel, descriptor
    launch, gather) and in 17 tokens (the batched path), both reduction
    modes, with and without the optional outputs: y, h and the index list of
    that token bitwise equal everywhere.  |u|, |g| <= 256 and at most 200
    intermediate entries, so h and y stay exact integers in fp32."""
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    rng = np.random.default_rng(5 + len(act))
    d, f = 128, 200
    k_in, k_mid = 51, 80
    wu = to_dev(np.ascontiguousarray(_ints(rng, (f, d), -1, 1).T), bf)
    wd = to_dev(np.ascontiguousarray(_ints(rng, (d, f), -1, 1).T), bf)
    kw = {}
    a = qs.ACT_RELU2
    if act == "glu":
        # |g| <= 2 * 128 / 4 keeps relu(g)^2 * u below 2^24 / 200
        kw["w_gate"] = to_dev(np.ascontiguousarray(_ints(rng, (f, d), 0, 0).T +
                                                   (rng.random((d, f)) < 0.1)), bf)
        a = qs.ACT_RELU2_GLU
    tok = _ints(rng, (1, d), -2, 2)
    outs = {}
    for det in (False, True):
        with reduction_mode(qs, det):
            for rows, pos in ((1, 0), (3, 1), (17, 16)):
                x = _batch_with(tok[0], _ints(rng, (rows, d), -2, 2), pos)
                for full in (False, True):
                    note(f"paths ffn {act} rows={rows} det={det} outputs={full}")
                    y, h, mi, mc = qs.qs_sparse_ffn(to_dev(x, bf), a, k_in, k_mid, wu, wd,
                                                    want_h=full, want_mid=full, **kw)
                    torch.cuda.synchronize()
                    outs[(rows, det, full)] = (y[pos].cpu().numpy(),
                                               h[pos].cpu().numpy() if full else None,
                                               mi[pos, :k_mid].cpu().numpy() if full else None)
    ry, rh, ri = outs[(1, True, True)]
    for key, (y, h, mi) in outs.items():
        assert np.array_equal(y.view(np.uint32), ry.view(np.uint32)), f"y differs on path {key}"
        if h is not None:
            assert np.array_equal(h.view(np.uint32), rh.view(np.uint32)), f"h differs on path {key}"
            assert np.array_equal(mi, ri), f"index list differs on path {key}"


def test_paths_i8t(gpu_lib):
    """Ternary x int8: each row alone and inside 7- and 16-row batches (the
    fused one-launch kernel, the split gather, the int8 matrix-core kernel):
    acc and y bitwise equal (int32 sums)."""
    import torch
    qs = gpu_lib
    rng = np.random.default_rng(6)
    d, n, k = 4096, 4096, 1587
    t, alpha = qs.qs_ternarize(datagen.normal(rng, (n, d), 0.02))
    wp = to_dev(qs.qs_pack_ternary(t))
    x16 = datagen.student_t(rng, (16, d))
    note("paths i8t 16 rows")
    acc16, y16, *_ = qs.qs_sparse_linear_i8t(to_dev(x16), k, wp, alpha, n)
    note("paths i8t 7 rows")
    acc7, y7, *_ = qs.qs_sparse_linear_i8t(to_dev(x16[:7]), k, wp, alpha, n)
    torch.cuda.synchronize()
    for r in (0, 3, 6):
        note(f"paths i8t row {r} alone")
        acc1, y1, *_ = qs.qs_sparse_linear_i8t(to_dev(x16[r:r + 1]), k, wp, alpha, n)
        torch.cuda.synchronize()
        for acc_b, y_b in ((acc16, y16), (acc7, y7)):
            assert np.array_equal(acc1[0].cpu().numpy(), acc_b[r].cpu().numpy())
            assert np.array_equal(y1[0].cpu().numpy().view(np.uint32), y_b[r].cpu().numpy().view(np.uint32))
