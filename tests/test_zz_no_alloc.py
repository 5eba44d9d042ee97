"""The allocation-free FFN entry point, qs_sparse_ffn_static, called through
the C ABI and checked against qs_sparse_ffn with a caller workspace: two
calls in a row, the second with a smaller batch (the shared per-GPU scratch
keeps the first call's contents).

* fixed-order split-K sums: y, h and the index list of the intermediate
  selection are bitwise equal to those of the workspace entry point;
* the default (float-atomic) sums: the stages match the oracle as in the FFN
  parity tests (h within its propagated bound, the selection of h exact on
  the device's h, y within tol * T of the oracle's down projection).
"""
import numpy as np
import pytest

import datagen
import oracle
from gpu_util import assert_within, note, reduction_mode, to_dev

pytestmark = pytest.mark.gpu

TOL = 4e-3


def _relu2_inputs(glu, batch, rotation):
    gen = datagen.c2g_relu2glu_ffn if glu else datagen.c2_relu2_ffn
    return gen(batch, rotation=rotation, with_weights=False)["X"]


def _calls(qs, act, x, k_in, k_mid, wu, wd, wg=None, bg=None, bu=None):
    import torch
    kw = dict(w_gate=wg, b_gate=bg, b_up=bu, want_h=True, want_mid=True)
    ys, hs, ms, cs = qs.qs_sparse_ffn_static(x, act, k_in, k_mid, wu, wd, **kw)
    yw, hw, mw, cw = qs.qs_sparse_ffn(x, act, k_in, k_mid, wu, wd, **kw)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in (ys, hs, ms, cs, yw, hw, mw, cw)]


@pytest.mark.parametrize("glu", [False, True])
def test_static_relu2_kinds_match_workspace_entry(gpu_lib, glu):
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    c = datagen.c2g_relu2glu_ffn(4) if glu else datagen.c2_relu2_ffn(4)
    k_in, k_mid = c["K_in"], c["K_mid"]
    wu = to_dev(np.ascontiguousarray(c["W_up"].T), bf)
    wd = to_dev(np.ascontiguousarray(c["W_down"].T), bf)
    wg = to_dev(np.ascontiguousarray(c["W_gate"].T), bf) if glu else None
    act = qs.ACT_RELU2_GLU if glu else qs.ACT_RELU2
    for batch, rot in ((4, 0), (1, 1)):
        x = _relu2_inputs(glu, batch, rot)
        xd = to_dev(x, bf)
        note(f"static FFN glu={glu} B={batch}: fixed-order sums")
        with reduction_mode(qs, True):
            ys, hs, ms, cs, yw, hw, mw, cw = _calls(qs, act, xd, k_in, k_mid, wu, wd, wg)
        assert np.array_equal(ys.view(np.uint32), yw.view(np.uint32))
        assert np.array_equal(hs.view(np.uint32), hw.view(np.uint32))
        assert np.array_equal(cs, cw)
        for r in range(batch):
            assert np.array_equal(ms[r, :cs[r]], mw[r, :cw[r]])
        note(f"static FFN glu={glu} B={batch}: atomic sums against the oracle")
        with reduction_mode(qs, False):
            ys, hs, ms, cs = [a.cpu().numpy() for a in qs.qs_sparse_ffn_static(
                xd, act, k_in, k_mid, wu, wd, w_gate=wg, want_h=True, want_mid=True)]
        if glu:
            ref = oracle.ffn_relu2_glu(x, k_in, c["W_gate"], c["W_up"], k_mid, c["W_down"])
            dg, du = TOL * ref["T_g"], TOL * ref["T_u"]
            rg = np.maximum(ref["g"], 0.0)
            bound = (2 * rg * dg + dg * dg) * (np.abs(ref["u"]) + du) + rg * rg * du
        else:
            ref = oracle.ffn_relu2(x, k_in, c["W_up"], k_mid, c["W_down"])
            bound = TOL * (2 * np.abs(ref["u"]) * ref["T_u"] + TOL * ref["T_u"] ** 2)
        assert np.all(np.abs(hs.astype(np.float64) - ref["h"]) <= bound)
        down = oracle.ffn_relu2_down_from(hs, k_mid, c["W_down"])
        for r in range(batch):
            assert cs[r] == k_mid and np.array_equal(ms[r, :k_mid], down["idx2"][r])
        assert_within(ys, down["y"], down["T_y"], TOL, "static FFN y")


def test_static_drelu_matches_workspace_entry(gpu_lib):
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    c = datagen.c5_drelu_ffn(4)
    d = c["X"].shape[1]
    wg, wu = to_dev(c["W_gate"], bf), to_dev(c["W_up"], bf)
    wd = to_dev(np.ascontiguousarray(c["W_down"].T), bf)
    bg, bu = to_dev(c["b_gate"]), to_dev(c["b_up"])
    for batch, rot in ((4, 0), (1, 1)):
        x = datagen.c5_drelu_ffn(batch, rotation=rot, with_weights=False)["X"]
        xd = to_dev(x, bf)
        note(f"static dReLU FFN B={batch}: fixed-order sums")
        with reduction_mode(qs, True):
            ys, hs, ms, cs, yw, hw, mw, cw = _calls(qs, qs.ACT_DRELU, xd, d, -1, wu, wd, wg, bg, bu)
        assert np.array_equal(ys.view(np.uint32), yw.view(np.uint32))
        assert np.array_equal(hs.view(np.uint32), hw.view(np.uint32))
        assert np.array_equal(cs, cw)
        note(f"static dReLU FFN B={batch}: atomic sums against the oracle")
        with reduction_mode(qs, False):
            ys, hs, ms, cs = [a.cpu().numpy() for a in qs.qs_sparse_ffn_static(
                xd, qs.ACT_DRELU, d, -1, wu, wd, w_gate=wg, b_gate=bg, b_up=bu, want_h=True,
                want_mid=True)]
        ref = oracle.ffn_drelu(x, c["W_gate"], c["b_gate"], c["W_up"], c["b_up"], c["W_down"])
        gp, up = np.maximum(ref["g"], 0), np.maximum(ref["u"], 0)
        bound = TOL * (ref["T_g"] * up + ref["T_u"] * gp + TOL * ref["T_g"] * ref["T_u"])
        assert np.all(np.abs(hs.astype(np.float64) - ref["h"]) <= bound)
        down = oracle.ffn_drelu_down_from(hs, c["W_down"])
        for r in range(batch):
            assert cs[r] == down["nz_count"][r]
            assert np.array_equal(ms[r, :cs[r]], down["nz_idx"][r])
        assert_within(ys, down["y"], down["T_y"], TOL, "static dReLU y")


def test_static_rejects_shapes_beyond_its_scratch(gpu_lib):
    """64 tokens of the Llama-7B FFN need a 52 MiB workspace: rejected
    before anything is enqueued (y keeps its contents)."""
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    x = torch.zeros((64, 4096), dtype=bf, device="cuda")
    wu = torch.zeros((4096, 11008), dtype=bf, device="cuda")
    wd = torch.zeros((11008, 4096), dtype=bf, device="cuda")
    y = torch.full((64, 4096), 3.0, dtype=torch.float32, device="cuda")
    note("static FFN: shape beyond the scratch")
    with pytest.raises(qs.QSError) as e:
        qs.qs_sparse_ffn_static(x, qs.ACT_RELU2, 1638, 4403, wu, wd, y=y)
    assert e.value.status == qs.QS_ERR_UNSUPPORTED and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
