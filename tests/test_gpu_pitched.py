"""GPU parity of padded weight rows (a row pitch wider than the row): the
squared-ReLU FFNs at 1-16 tokens, the dReLU FFN's down gather, the sparse
linear and the selection-in-gather read the rows of W^T ldw elements apart
and never touch the padding.

Every padding column holds NaN, so a read of it would show in y.  The padded
call reads the same numbers in the same order as the unpadded call (only the
addresses differ), so:

* with fixed-order split-K sums, y (and h) of the padded call are bitwise
  equal to those of the unpadded call, at the Llama-7B shape and at a small
  ragged one, for pads of 8 and 64 columns;
* in the default accumulate form (float atomics), y is within the fp32
  summation bound of the unpadded call and within the bf16 tolerance of the
  oracle's down projection of h (Turbo Sparse summary, Eq. 3-4: the top-k% of
  h by |h| before W_down);
* the one-token linear (Q-Sparse news article, Top-K section) is bitwise equal
  in both modes (one launch, fixed-order sums);
* qs_topk_gather_linear_acc is within the fp32 bound of the oracle.
"""
import numpy as np
import pytest

import datagen
import oracle
from gpu_util import assert_within, note, reduction_mode, to_dev

pytestmark = pytest.mark.gpu

TOL_BF16 = 4e-3
SUM_EPS = 1e-5


def _padded(a, pad, dtype):
    """Device copy of the 2-D array `a` whose rows are len + pad apart, the
    padding NaN; returned as the [rows, len] view."""
    import torch
    r, c = a.shape
    t = torch.full((r, c + pad), float("nan"), dtype=dtype, device="cuda")
    t[:, :c] = to_dev(a, dtype)
    v = t[:, :c]
    assert v.stride() == (c + pad, 1)
    return v


def _small(seed):
    rng = np.random.default_rng(seed)
    d, f = 520, 1368
    x = datagen.bf16_round(datagen.student_t(rng, (1, d)))
    w_up = datagen.bf16_round(datagen.normal(rng, (f, d), 0.02))
    w_gate = datagen.bf16_round(datagen.normal(rng, (f, d), 0.02))
    w_down = datagen.bf16_round(datagen.normal(rng, (d, f), 0.02))
    return {"X": x, "W_up": w_up, "W_gate": w_gate, "W_down": w_down,
            "K_in": (2 * d) // 5, "K_mid": (2 * f) // 5}


def _cases():
    c = datagen.c2_relu2_ffn(1)
    return [("llama7b", c), ("small", _small(71))]


@pytest.mark.parametrize("pad", [8, 64])
@pytest.mark.parametrize("glu", [False, True])
def test_pitched_ffn_one_token(gpu_lib, pad, glu):
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    for name, c in _cases():
        if glu and "W_gate" not in c:
            rng = np.random.default_rng(5)
            c = dict(c, W_gate=datagen.bf16_round(datagen.normal(rng, c["W_up"].shape, 0.02)))
        act = qs.ACT_RELU2_GLU if glu else qs.ACT_RELU2
        x, k_in, k_mid = c["X"], c["K_in"], c["K_mid"]
        wu_t, wd_t = np.ascontiguousarray(c["W_up"].T), np.ascontiguousarray(c["W_down"].T)
        wg_t = np.ascontiguousarray(c["W_gate"].T) if glu else None
        xd = to_dev(x, bf)
        nat = dict(w_up=to_dev(wu_t, bf), w_down_t=to_dev(wd_t, bf),
                   w_gate=to_dev(wg_t, bf) if glu else None)
        pad_w = dict(w_up=_padded(wu_t, pad, bf), w_down_t=_padded(wd_t, pad, bf),
                     w_gate=_padded(wg_t, pad, bf) if glu else None)
        note(f"pitched FFN {name} glu={glu} pad={pad}")
        with reduction_mode(qs, True):
            y0, h0, _, _ = qs.qs_sparse_ffn(xd, act, k_in, k_mid, nat["w_up"], nat["w_down_t"],
                                            w_gate=nat["w_gate"], want_h=True)
            y1, h1, _, _ = qs.qs_sparse_ffn(xd, act, k_in, k_mid, pad_w["w_up"], pad_w["w_down_t"],
                                            w_gate=pad_w["w_gate"], want_h=True)
            torch.cuda.synchronize()
        y0, y1 = y0.cpu().numpy(), y1.cpu().numpy()
        assert np.array_equal(h0.cpu().numpy().view(np.uint32), h1.cpu().numpy().view(np.uint32))
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), f"{name}: fixed-order y differs"
        # the default accumulate form, against the unpadded call and the oracle
        h = h0.cpu().numpy()
        down = oracle.ffn_relu2_down_from(h, k_mid, c["W_down"])
        with reduction_mode(qs, False):
            y2, _, _, _ = qs.qs_sparse_ffn(xd, act, k_in, k_mid, pad_w["w_up"], pad_w["w_down_t"],
                                           w_gate=pad_w["w_gate"])
            torch.cuda.synchronize()
        y2 = y2.cpu().numpy()
        assert np.all(np.isfinite(y2))
        assert_within(y2, y0.astype(np.float64), down["T_y"], 2 * SUM_EPS, f"{name}: atomic vs fixed")
        assert_within(y2, down["y"], down["T_y"], TOL_BF16, f"{name}: atomic vs oracle")


@pytest.mark.parametrize("pad", [8, 64])
def test_pitched_linear_one_token(gpu_lib, pad):
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    for name, c in _cases():
        x, k = c["X"], c["K_in"]
        wt = np.ascontiguousarray(c["W_up"].T)
        xd = to_dev(x, bf)
        for det in (True, False):
            note(f"pitched linear {name} pad={pad} det={det}")
            with reduction_mode(qs, det):
                y0 = qs.qs_sparse_linear(xd, k, to_dev(wt, bf))
                y1 = qs.qs_sparse_linear(xd, k, _padded(wt, pad, bf))
                torch.cuda.synchronize()
            assert np.array_equal(y0.cpu().numpy().view(np.uint32), y1.cpu().numpy().view(np.uint32))
        mask, _, _, _ = oracle.topk_select(oracle.magnitude(x), k)
        y_ref, t = oracle.sparse_linear(x, c["W_up"], mask)
        assert_within(y1.cpu().numpy(), y_ref, t, TOL_BF16, f"{name}: pitched linear vs oracle")


@pytest.mark.parametrize("pad", [8, 64])
def test_pitched_topk_gather(gpu_lib, pad):
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    rng = np.random.default_rng(300 + pad)
    for d_in, n_out in ((11008, 4096), (1368, 520)):
        x = datagen.student_t(rng, (2, d_in)).astype(np.float32)
        w = datagen.bf16_round(datagen.normal(rng, (n_out, d_in), 0.02))
        k = (2 * d_in) // 5
        note(f"pitched topk-gather {d_in}x{n_out} pad={pad}")
        y = torch.zeros((2, n_out), dtype=torch.float32, device="cuda")
        qs.qs_topk_gather_linear_acc(to_dev(x), k, _padded(np.ascontiguousarray(w.T), pad, bf), y)
        torch.cuda.synchronize()
        mask, _, _, _ = oracle.topk_select(oracle.magnitude(x), k)
        y_ref, t = oracle.sparse_linear(x, w, mask)
        assert_within(y.cpu().numpy(), y_ref, t, SUM_EPS, "pitched topk-gather vs oracle")


@pytest.mark.parametrize("rows", [2, 4, 8, 16])
@pytest.mark.parametrize("glu", [False, True])
def test_pitched_ffn_batches(gpu_lib, rows, glu):
    """2-16 tokens (the selection launch, the column kernel or the gathers,
    the 16-token matrix-core gather): fixed-order y bitwise equal to the
    unpadded call's, NaN padding never read."""
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    for d, f in ((4096, 11008), (520, 1368)):
        c = (datagen.c2g_relu2glu_ffn if glu else datagen.c2_relu2_ffn)(rows, d=d, ffn=f)
        act = qs.ACT_RELU2_GLU if glu else qs.ACT_RELU2
        wu_t, wd_t = np.ascontiguousarray(c["W_up"].T), np.ascontiguousarray(c["W_down"].T)
        wg_t = np.ascontiguousarray(c["W_gate"].T) if glu else None
        xd = to_dev(c["X"], bf)
        note(f"pitched FFN rows={rows} glu={glu} {d}x{f}")
        with reduction_mode(qs, True):
            y0, _, _, _ = qs.qs_sparse_ffn(xd, act, c["K_in"], c["K_mid"], to_dev(wu_t, bf),
                                           to_dev(wd_t, bf),
                                           w_gate=to_dev(wg_t, bf) if glu else None)
            y1, _, _, _ = qs.qs_sparse_ffn(xd, act, c["K_in"], c["K_mid"], _padded(wu_t, 64, bf),
                                           _padded(wd_t, 64, bf),
                                           w_gate=_padded(wg_t, 64, bf) if glu else None)
            torch.cuda.synchronize()
        y0, y1 = y0.cpu().numpy(), y1.cpu().numpy()
        assert np.all(np.isfinite(y1))
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), f"rows={rows} {d}x{f}"


@pytest.mark.parametrize("rows", [1, 4, 16])
def test_pitched_drelu_down(gpu_lib, rows):
    """dReLU with W_down^T rows padded (W_gate and W_up natural): fixed-order y
    bitwise equal to the unpadded call's."""
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    c = datagen.c5_drelu_ffn(rows, d=1024, ffn=3584)
    wd_t = np.ascontiguousarray(c["W_down"].T)
    xd = to_dev(c["X"], bf)
    kw = dict(w_gate=to_dev(c["W_gate"], bf), b_gate=to_dev(c["b_gate"]), b_up=to_dev(c["b_up"]))
    note(f"pitched dReLU rows={rows}")
    with reduction_mode(qs, True):
        y0, _, _, _ = qs.qs_sparse_ffn(xd, qs.ACT_DRELU, 1024, -1, to_dev(c["W_up"], bf),
                                       to_dev(wd_t, bf), **kw)
        y1, _, _, _ = qs.qs_sparse_ffn(xd, qs.ACT_DRELU, 1024, -1, to_dev(c["W_up"], bf),
                                       _padded(wd_t, 64, bf), **kw)
        torch.cuda.synchronize()
    y0, y1 = y0.cpu().numpy(), y1.cpu().numpy()
    assert np.all(np.isfinite(y1))
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))


@pytest.mark.parametrize("rows", [3, 8, 16])
def test_pitched_linear_batches(gpu_lib, rows):
    """qs_sparse_linear on padded W^T rows through the selection launch and
    the gathers: fixed-order y bitwise equal to the unpadded call's."""
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    rng = np.random.default_rng(40 + rows)
    x = datagen.bf16_round(datagen.student_t(rng, (rows, 1536)))
    wt = np.ascontiguousarray(datagen.bf16_round(datagen.normal(rng, (1032, 1536), 0.02)).T)
    xd = to_dev(x, bf)
    note(f"pitched linear rows={rows}")
    with reduction_mode(qs, True):
        y0 = qs.qs_sparse_linear(xd, 614, to_dev(wt, bf))
        y1 = qs.qs_sparse_linear(xd, 614, _padded(wt, 64, bf))
        torch.cuda.synchronize()
    assert np.array_equal(y0.cpu().numpy().view(np.uint32), y1.cpu().numpy().view(np.uint32))


def test_pitched_drelu_up_rejected(gpu_lib):
    """dReLU with padded W_up rows: QS_ERR_UNSUPPORTED, nothing enqueued (y untouched)."""
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    c = datagen.c5_drelu_ffn(2, d=1024, ffn=3584)
    y = torch.full((2, 1024), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(qs.QSError) as e:
        qs.qs_sparse_ffn(to_dev(c["X"], bf), qs.ACT_DRELU, 1024, -1, _padded(c["W_up"], 8, bf),
                         to_dev(np.ascontiguousarray(c["W_down"].T), bf),
                         w_gate=_padded(c["W_gate"], 8, bf), b_gate=to_dev(c["b_gate"]),
                         b_up=to_dev(c["b_up"]), y=y)
    assert e.value.status == qs.QS_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
