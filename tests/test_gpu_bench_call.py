"""GPU parity of qs_sparse_ffn called exactly as the benchmark calls it:
h, mid_idx and mid_cnt NULL, fp32 y, the full workload shapes.

Without h or the index list the selection launches take other branches (no
write-back of h, no second block scan for the index list), so these calls are
checked on their own:

* fixed-order split-K sums: y of the bare call is bitwise equal to y of the
  same call with every optional output on, whose stages the FFN tests check
  against the oracle, where both calls run the same down gather (several
  tokens); with one token the bare call's down gather selects h itself, and
  its y is within the fp32 summation bound (1e-5 * T_y) of the oracle's down
  projection of the outputs-on call's h over the oracle's selection (h has
  no atomics: the same in both calls);
* the default accumulate form (float atomics, so the fp32 sums of two calls
  may differ in their last bits): y of the bare call is within tol * T_y of
  the oracle's down projection of h taken from an outputs-on call on the same
  inputs, plus an allowance for the intermediate entries whose selection a
  last-bit difference in h could flip (entries within twice the sum-order
  bound of the selection threshold); the number of such entries is printed.
  Q-Sparse's top-k on the intermediate: Turbo Sparse summary, Eq. 3-4 (top-k%
  by |h| before W_down).
"""
import numpy as np
import pytest

import datagen
import oracle
from gpu_util import assert_within, note, reduction_mode, to_dev

pytestmark = pytest.mark.gpu

TOL_BF16 = 4e-3
SUM_EPS = 1e-5    # bound of the fp32 summation of the gathers (fp32 tolerance)


def _bare_and_full(qs, act, xd, k_in, k_mid, wu, wd, wg=None, bg=None, bu=None):
    import torch
    kw = dict(w_gate=wg, b_gate=bg, b_up=bu)
    y_bare = torch.empty((xd.shape[0], wd.shape[1]), dtype=torch.float32, device=xd.device)
    qs.qs_sparse_ffn(xd, act, k_in, k_mid, wu, wd, y=y_bare, **kw)
    y_full, h, mid_idx, mid_cnt = qs.qs_sparse_ffn(xd, act, k_in, k_mid, wu, wd,
                                                   want_h=True, want_mid=True, **kw)
    torch.cuda.synchronize()
    return y_bare.cpu().numpy(), y_full.cpu().numpy(), h.cpu().numpy()


def _flip_allowance(h, dh, k_mid, w_down):
    """Entries whose top-k_mid membership a change of at most dh (per entry)
    in h could flip, and the bound on y that their flips and dh add."""
    mag = np.abs(h.astype(np.float64))
    aw = np.abs(w_down.astype(np.float64))
    allow = np.zeros((h.shape[0], w_down.shape[0]))
    n_flip = 0
    for r in range(h.shape[0]):
        near = np.zeros(mag.shape[1], dtype=bool)
        if k_mid > 0:
            # the k_mid-th largest entry (ties to the lower index) and its bound
            t = np.lexsort((np.arange(mag.shape[1]), -mag[r]))[k_mid - 1]
            near = np.abs(mag[r] - mag[r, t]) <= dh[r] + dh[r, t]
        n_flip += int(near.sum())
        allow[r] = aw[:, near] @ mag[r, near] + aw @ dh[r]
    return allow, n_flip


def _check_relu2(gpu_lib, c, glu=False):
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    x, k_in, k_mid = c["X"], c["K_in"], c["K_mid"]
    xd = to_dev(x, bf)
    wu = to_dev(np.ascontiguousarray(c["W_up"].T), bf)
    wd = to_dev(np.ascontiguousarray(c["W_down"].T), bf)
    wg = to_dev(np.ascontiguousarray(c["W_gate"].T), bf) if glu else None
    act = qs.ACT_RELU2_GLU if glu else qs.ACT_RELU2
    with reduction_mode(qs, True):
        y_bare, y_full, h_det = _bare_and_full(qs, act, xd, k_in, k_mid, wu, wd, wg)
    if x.shape[0] > 1:
        assert np.array_equal(y_bare.view(np.uint32), y_full.view(np.uint32)), \
            "fixed-order mode: bare call differs from the outputs-on call"
    else:
        down = oracle.ffn_relu2_down_from(h_det, k_mid, c["W_down"])
        assert_within(y_bare, down["y"], down["T_y"], SUM_EPS, "fixed-order bare call y")
    with reduction_mode(qs, False):
        y_bare, _, h = _bare_and_full(qs, act, xd, k_in, k_mid, wu, wd, wg)
    if glu:
        ref = oracle.ffn_relu2_glu(x, k_in, c["W_gate"], c["W_up"], k_mid, c["W_down"])
        dg, du = 2 * SUM_EPS * ref["T_g"], 2 * SUM_EPS * ref["T_u"]
        rg = np.maximum(ref["g"], 0.0)
        dh = (2 * rg * dg + dg * dg) * (np.abs(ref["u"]) + du) + rg * rg * du
    else:
        ref = oracle.ffn_relu2(x, k_in, c["W_up"], k_mid, c["W_down"])
        du = 2 * SUM_EPS * ref["T_u"]
        dh = 2 * np.abs(ref["u"]) * du + du * du
    down = oracle.ffn_relu2_down_from(h, k_mid, c["W_down"])
    allow, n_flip = _flip_allowance(h, dh, k_mid, c["W_down"])
    err = np.abs(y_bare.astype(np.float64) - down["y"])
    bound = TOL_BF16 * down["T_y"] + allow
    assert np.all(err <= bound), f"bare call y outside tol: worst excess {np.max(err - bound)}"
    rel = float(np.max(err / np.maximum(down["T_y"], 1e-300)))
    print(f"bare call: max |dy|/T_y = {rel:.2e}; intermediate entries near the threshold: {n_flip}")


@pytest.mark.parametrize("batch", [1, 16])
def test_bench_call_relu2_c2(gpu_lib, batch):
    note(f"bench call: relu2 FFN C2 B={batch}, h/mid NULL")
    _check_relu2(gpu_lib, datagen.c2_relu2_ffn(batch))


def test_bench_call_relu2_glu_c2g(gpu_lib):
    note("bench call: gated relu2 FFN Llama-7B shape B=1, h/mid NULL")
    _check_relu2(gpu_lib, datagen.c2g_relu2glu_ffn(1), glu=True)


@pytest.mark.parametrize("batch", [1, 4])
def test_bench_call_drelu_c5(gpu_lib, batch):
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    c = datagen.c5_drelu_ffn(batch)
    d = c["X"].shape[1]
    xd = to_dev(c["X"], bf)
    wg, wu = to_dev(c["W_gate"], bf), to_dev(c["W_up"], bf)
    wd = to_dev(np.ascontiguousarray(c["W_down"].T), bf)
    bg, bu = to_dev(c["b_gate"]), to_dev(c["b_up"])
    note(f"bench call: dReLU FFN C5 B={batch}, h/mid NULL")
    with reduction_mode(qs, True):
        y_bare, y_full, _ = _bare_and_full(qs, qs.ACT_DRELU, xd, d, -1, wu, wd, wg, bg, bu)
    assert np.array_equal(y_bare.view(np.uint32), y_full.view(np.uint32))
    with reduction_mode(qs, False):
        y_bare, _, h = _bare_and_full(qs, qs.ACT_DRELU, xd, d, -1, wu, wd, wg, bg, bu)
    # the gate/up sums are not split (no atomics), so h and its nonzero set
    # are the same in every call
    down = oracle.ffn_drelu_down_from(h, c["W_down"])
    assert_within(y_bare, down["y"], down["T_y"], TOL_BF16, "dReLU bare call y")
