"""GPU parity of the sparse FFNs, stage by stage.

The masks of the second stage are computed from floating-point intermediates,
so the contract is stage-wise:
  1. h_gpu is within the bound propagated from the up/gate tolerance:
       relu2:  tol * (2 |u_ref| T_u + tol T_u^2)
       dReLU:  tol * (T_g u_ref+ + T_u g_ref+ + tol T_g T_u)
  2. the selected intermediate entries equal the oracle's selection applied
     to h_gpu, exactly;
  3. y_gpu is within tol * T of the oracle's down projection of (h_gpu, that
     selection).
"""
import numpy as np
import pytest

import datagen
import oracle
from gpu_util import assert_within, note, reduction_mode, to_dev

pytestmark = pytest.mark.gpu


def _relu2_case(gpu_lib, x, w_up, w_down, k_in, k_mid, wtype="bf16", ydt=None):
    import torch
    qs = gpu_lib
    dt = torch.bfloat16 if wtype == "bf16" else torch.float32
    tol = 4e-3 if wtype == "bf16" else 1e-5
    y, h, mid_idx, mid_cnt = qs.qs_sparse_ffn(
        to_dev(x, dt), qs.ACT_RELU2, k_in, k_mid, to_dev(np.ascontiguousarray(w_up.T), dt),
        to_dev(np.ascontiguousarray(w_down.T), dt), y_dtype=ydt or torch.float32,
        want_h=True, want_mid=True)
    torch.cuda.synchronize()
    y, h, mid_idx, mid_cnt = (a.float().cpu().numpy() if a.dtype == torch.bfloat16 else
                              a.cpu().numpy() for a in (y, h, mid_idx, mid_cnt))
    ref = oracle.ffn_relu2(x, k_in, w_up, k_mid if k_mid >= 0 else w_up.shape[0], w_down)
    bound = tol * (2 * np.abs(ref["u"]) * ref["T_u"] + tol * ref["T_u"] ** 2)
    err = np.abs(h.astype(np.float64) - ref["h"])
    assert np.all(err <= bound), f"h outside bound: worst {np.max(err - bound)}"
    if k_mid >= 0:
        down = oracle.ffn_relu2_down_from(h, k_mid, w_down)
        for r in range(x.shape[0]):
            assert mid_cnt[r] == k_mid
            assert np.array_equal(mid_idx[r, :k_mid], down["idx2"][r])
    else:
        down = oracle.ffn_drelu_down_from(h, w_down)
        for r in range(x.shape[0]):
            assert mid_cnt[r] == down["nz_count"][r]
            assert np.array_equal(mid_idx[r, :mid_cnt[r]], down["nz_idx"][r])
    assert_within(y, down["y"], down["T_y"], tol, "relu2 y")
    flips = int(np.sum(down.get("mask2", down.get("nz_mask")) != ref["mask2"])) if k_mid >= 0 else 0
    return flips


@pytest.mark.parametrize("rows,d,f", [(1, 64, 96), (3, 256, 520), (17, 512, 264)])
@pytest.mark.parametrize("wtype", ["f32", "bf16"])
@pytest.mark.parametrize("det", [False, True])
def test_relu2_small(gpu_lib, rows, d, f, wtype, det):
    """det: fixed-order split-K sums; else the accumulate forms (the
    selections clear the sums, the selection of h applies relu^2)."""
    rng = np.random.default_rng(rows + d + f)
    x = datagen.student_t(rng, (rows, d))
    w_up = datagen.normal(rng, (f, d), 0.02)
    w_down = datagen.normal(rng, (d, f), 0.02)
    if wtype == "bf16":
        x, w_up, w_down = (datagen.bf16_round(a) for a in (x, w_up, w_down))
    with reduction_mode(gpu_lib, det):
        for k_in, k_mid in [(d, f), ((2 * d) // 5, (2 * f) // 5), (1, 3), (0, 0), (d // 2, -1)]:
            note(f"relu2 {wtype} det={det} rows={rows} d={d} ffn={f} k_in={k_in} k_mid={k_mid}")
            _relu2_case(gpu_lib, x, w_up, w_down, k_in, k_mid, wtype)


@pytest.mark.parametrize("batch", [1, 2, 4, 8, 16])
def test_relu2_full_c2(gpu_lib, batch):
    c = datagen.c2_relu2_ffn(batch)
    note(f"relu2 FFN full config C2 B={batch}")
    flips = _relu2_case(gpu_lib, c["X"], c["W_up"], c["W_down"], c["K_in"], c["K_mid"])
    print(f"C2 B={batch}: end-to-end mask entries differing from the oracle's own: {flips}")


def test_relu2_bf16_output(gpu_lib):
    import torch
    c = datagen.c2_relu2_ffn(2)
    note("relu2 FFN C2 B=2 bf16 output")
    _relu2_case(gpu_lib, c["X"], c["W_up"], c["W_down"], c["K_in"], c["K_mid"],
                ydt=torch.bfloat16)


# ---------------------------------------------------------------- gated squared ReLU

def _relu2_glu_case(gpu_lib, x, wg, wu, wd, k_in, k_mid, wtype="bf16"):
    import torch
    qs = gpu_lib
    dt = torch.bfloat16 if wtype == "bf16" else torch.float32
    tol = 4e-3 if wtype == "bf16" else 1e-5
    f = wu.shape[0]
    y, h, mid_idx, mid_cnt = qs.qs_sparse_ffn(
        to_dev(x, dt), qs.ACT_RELU2_GLU, k_in, k_mid, to_dev(np.ascontiguousarray(wu.T), dt),
        to_dev(np.ascontiguousarray(wd.T), dt), w_gate=to_dev(np.ascontiguousarray(wg.T), dt),
        want_h=True, want_mid=True)
    torch.cuda.synchronize()
    y, h, mid_idx, mid_cnt = (a.cpu().numpy() for a in (y, h, mid_idx, mid_cnt))
    ref = oracle.ffn_relu2_glu(x, k_in, wg, wu, k_mid if k_mid >= 0 else f, wd)
    # h = relu(g)^2 u with g, u each within tol * T: relu is 1-Lipschitz, so
    # |dh| <= (2 relu(g) dg + dg^2)(|u| + du) + relu(g)^2 du.
    dg, du = tol * ref["T_g"], tol * ref["T_u"]
    rg = np.maximum(ref["g"], 0.0)
    bound = (2 * rg * dg + dg * dg) * (np.abs(ref["u"]) + du) + rg * rg * du
    err = np.abs(h.astype(np.float64) - ref["h"])
    assert np.all(err <= bound), f"h outside bound: worst {np.max(err - bound)}"
    if k_mid >= 0:
        down = oracle.ffn_relu2_down_from(h, k_mid, wd)
        for r in range(x.shape[0]):
            assert mid_cnt[r] == k_mid
            assert np.array_equal(mid_idx[r, :k_mid], down["idx2"][r])
    else:
        down = oracle.ffn_drelu_down_from(h, wd)
        for r in range(x.shape[0]):
            assert mid_cnt[r] == down["nz_count"][r]
            assert np.array_equal(mid_idx[r, :mid_cnt[r]], down["nz_idx"][r])
    assert_within(y, down["y"], down["T_y"], tol, "relu2-glu y")


@pytest.mark.parametrize("rows,d,f", [(1, 64, 96), (2, 128, 200), (3, 256, 520), (17, 512, 264)])
@pytest.mark.parametrize("wtype", ["f32", "bf16"])
@pytest.mark.parametrize("det", [False, True])
def test_relu2_glu_small(gpu_lib, rows, d, f, wtype, det):
    rng = np.random.default_rng(rows + 2 * d + f)
    x = datagen.student_t(rng, (rows, d))
    wg = datagen.normal(rng, (f, d), 0.02)
    wu = datagen.normal(rng, (f, d), 0.02)
    wd = datagen.normal(rng, (d, f), 0.02)
    if wtype == "bf16":
        x, wg, wu, wd = (datagen.bf16_round(a) for a in (x, wg, wu, wd))
    with reduction_mode(gpu_lib, det):
        for k_in, k_mid in [(d, f), ((2 * d) // 5, (2 * f) // 5), (1, 3), (0, 0), (d // 2, -1)]:
            note(f"relu2-glu {wtype} det={det} rows={rows} d={d} ffn={f} k_in={k_in} k_mid={k_mid}")
            _relu2_glu_case(gpu_lib, x, wg, wu, wd, k_in, k_mid, wtype)


@pytest.mark.parametrize("batch", [1, 4, 8, 16])
def test_relu2_glu_full_llama7b(gpu_lib, batch):
    c = datagen.c2g_relu2glu_ffn(batch)
    note(f"gated relu2 FFN, Llama-7B shape, B={batch}")
    _relu2_glu_case(gpu_lib, c["X"], c["W_gate"], c["W_up"], c["W_down"], c["K_in"], c["K_mid"])


# ---------------------------------------------------------------- dReLU

def _drelu_case(gpu_lib, x, wg, bg, wu, bu, wd, k_in=None, k_mid=-1):
    import torch
    qs = gpu_lib
    d = x.shape[1]
    k_in = d if k_in is None else k_in
    bf = torch.bfloat16
    y, h, mid_idx, mid_cnt = qs.qs_sparse_ffn(
        to_dev(x, bf), qs.ACT_DRELU, k_in, k_mid, to_dev(wu, bf),
        to_dev(np.ascontiguousarray(wd.T), bf), w_gate=to_dev(wg, bf),
        b_gate=None if bg is None else to_dev(bg), b_up=None if bu is None else to_dev(bu),
        want_h=True, want_mid=True)
    torch.cuda.synchronize()
    y, h, mid_idx, mid_cnt = (a.cpu().numpy() for a in (y, h, mid_idx, mid_cnt))
    xm = x
    if k_in < d:
        m1, _, _, _ = oracle.topk_select(oracle.magnitude(x), k_in)
        xm = np.where(m1 == 1, x, 0.0)
    ref = oracle.ffn_drelu(xm, wg, bg, wu, bu, wd)
    tol = 4e-3
    gp, up = np.maximum(ref["g"], 0), np.maximum(ref["u"], 0)
    bound = tol * (ref["T_g"] * up + ref["T_u"] * gp + tol * ref["T_g"] * ref["T_u"])
    err = np.abs(h.astype(np.float64) - ref["h"])
    assert np.all(err <= bound), f"h outside bound: worst {np.max(err - bound)}"
    if k_mid < 0:
        down = oracle.ffn_drelu_down_from(h, wd)
        for r in range(x.shape[0]):
            assert mid_cnt[r] == down["nz_count"][r]
            assert np.array_equal(mid_idx[r, :mid_cnt[r]], down["nz_idx"][r])
    else:
        down = oracle.ffn_relu2_down_from(h, k_mid, wd)
        for r in range(x.shape[0]):
            assert mid_cnt[r] == k_mid and np.array_equal(mid_idx[r, :k_mid], down["idx2"][r])
    assert_within(y, down["y"], down["T_y"], tol, "drelu y")
    return float(np.mean(h == 0))


@pytest.mark.parametrize("rows,d,f", [(1, 64, 48), (3, 256, 520), (4, 200, 136), (16, 512, 264),
                                      (21, 200, 136)])
@pytest.mark.parametrize("det", [False, True])
def test_drelu_small(gpu_lib, rows, d, f, det):
    rng = np.random.default_rng(rows * 5 + d + f)
    x = datagen.bf16_round(datagen.student_t(rng, (rows, d)))
    wg = datagen.bf16_round(datagen.normal(rng, (f, d), 0.02))
    wu = datagen.bf16_round(datagen.normal(rng, (f, d), 0.02))
    wd = datagen.bf16_round(datagen.normal(rng, (d, f), 0.02))
    bg = rng.normal(-0.2, 0.1, size=f).astype(np.float32)
    bu = rng.normal(-0.2, 0.1, size=f).astype(np.float32)
    with reduction_mode(gpu_lib, det):
        note(f"drelu det={det} rows={rows} d={d} ffn={f} (biases)")
        _drelu_case(gpu_lib, x, wg, bg, wu, bu, wd)
        note(f"drelu det={det} rows={rows} d={d} ffn={f} (no biases, top-K on x and on h)")
        _drelu_case(gpu_lib, x, wg, None, wu, None, wd, k_in=d // 2, k_mid=f // 3)


@pytest.mark.parametrize("batch", [1, 4, 16])
def test_drelu_full_c5(gpu_lib, batch):
    c = datagen.c5_drelu_ffn(batch)
    note(f"dReLU FFN full config C5 B={batch}")
    zero = _drelu_case(gpu_lib, c["X"], c["W_gate"], c["b_gate"], c["W_up"], c["b_up"],
                       c["W_down"])
    print(f"C5 B={batch}: zero fraction of h = {zero:.3f}")
    assert 0.8 < zero < 0.97
