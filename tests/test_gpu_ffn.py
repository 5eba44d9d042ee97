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
from gpu_util import assert_within, note, to_dev

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
def test_relu2_small(gpu_lib, rows, d, f, wtype):
    rng = np.random.default_rng(rows + d + f)
    x = datagen.student_t(rng, (rows, d))
    w_up = datagen.normal(rng, (f, d), 0.02)
    w_down = datagen.normal(rng, (d, f), 0.02)
    if wtype == "bf16":
        x, w_up, w_down = (datagen.bf16_round(a) for a in (x, w_up, w_down))
    for k_in, k_mid in [(d, f), ((2 * d) // 5, (2 * f) // 5), (1, 3), (0, 0), (d // 2, -1)]:
        note(f"relu2 {wtype} rows={rows} d={d} ffn={f} k_in={k_in} k_mid={k_mid}")
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
