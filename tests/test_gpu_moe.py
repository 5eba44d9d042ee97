"""GPU parity of the mixture-of-experts dReLU FFN (qs_sparse_moe_ffn), checked
stage by stage like the dense dReLU FFN, since the routing and the nonzero
sets are decisions taken on floating-point values:

  1. router logits within 1e-5 * T (fp32 sums of exact bf16 products,
     T = |x| . |W_router|^T);
  2. the chosen experts equal the oracle's top-k applied to the GPU's logits,
     and their weights the softmax of those logits (fp32: 1e-6 relative);
  3. each pair's h within the propagated bound
     tol * (T_g u+ + T_u g+ + tol T_g T_u), tol = 4e-3 (bf16 inputs);
  4. y within tol * T of the oracle's down projections of the GPU's h,
     combined with the GPU's weights.
"""
import numpy as np
import pytest

import datagen
import oracle
from gpu_util import note, reduction_mode, to_dev

pytestmark = pytest.mark.gpu


def _moe_case(qs, c, top_k, ydt=None):
    import torch
    bf = torch.bfloat16
    y, logits, experts, weights, h = qs.qs_sparse_moe_ffn(
        to_dev(c["X"], bf), top_k, to_dev(c["W_router"], bf), to_dev(c["W_gate"], bf),
        to_dev(c["W_up"], bf), to_dev(c["W_down_t"], bf), b_gate=to_dev(c["b_gate"]),
        b_up=to_dev(c["b_up"]), y_dtype=ydt or torch.float32, want_all=True)
    torch.cuda.synchronize()
    y, logits, experts, weights, h = (a.float().cpu().numpy() if a.dtype == bf else a.cpu().numpy()
                                      for a in (y, logits, experts, weights, h))
    x = c["X"]
    lg_ref, _, _, t_lg = oracle.moe_route(x, c["W_router"], top_k)
    assert np.all(np.abs(logits - lg_ref) <= 1e-5 * t_lg)
    # routing decided on the GPU's own logits
    rows, e = logits.shape
    for r in range(rows):
        order = np.lexsort((np.arange(e), -logits[r].astype(np.float64)))
        sel = np.sort(order[:top_k])
        assert experts[r].tolist() == sel.tolist()
        z = np.exp(logits[r, sel].astype(np.float64) - logits[r, sel].max())
        assert np.allclose(weights[r], z / z.sum(), rtol=1e-6, atol=0)
    w_down = np.transpose(c["W_down_t"], (0, 2, 1))
    ref = oracle.moe_drelu_ffn(x, c["W_router"], top_k, c["W_gate"], c["b_gate"], c["W_up"],
                               c["b_up"], w_down, experts=experts, weights=weights)
    tol = 4e-3
    gp, up = np.maximum(ref["g"], 0), np.maximum(ref["u"], 0)
    bound = tol * (ref["T_g"] * up + ref["T_u"] * gp + tol * ref["T_g"] * ref["T_u"])
    err = np.abs(h.astype(np.float64) - ref["h"])
    assert np.all(err <= bound), f"h outside bound: worst {np.max(err - bound)}"
    # the down projections of the GPU's h, combined with the GPU's weights
    y_ref = np.zeros_like(ref["y"])
    t_ref = np.zeros_like(ref["y"])
    for r in range(rows):
        for j in range(top_k):
            dn = oracle.ffn_drelu_down_from(h[r, j][None, :], w_down[experts[r, j]])
            y_ref[r] += weights[r, j] * dn["y"][0]
            t_ref[r] += abs(weights[r, j]) * dn["T_y"][0]
    err = np.abs(y.astype(np.float64) - y_ref)
    assert np.all(err <= tol * t_ref + 1e-30), f"y outside tol*T: worst {np.max(err - tol * t_ref)}"
    return float(np.mean(h == 0))


@pytest.mark.parametrize("rows,d,ffn,e,k", [(1, 256, 512, 8, 2), (3, 256, 520, 8, 2),
                                            (16, 512, 264, 8, 2), (5, 128, 136, 4, 1),
                                            (4, 64, 48, 6, 3), (12, 128, 136, 2, 1)])
@pytest.mark.parametrize("det", [False, True])
def test_moe_small(gpu_lib, rows, d, ffn, e, k, det):
    """det: fixed-order sums and the combine launch; else each pair's down
    gather adds weight * partial straight into its token's row of y."""
    sigma = 0.02 * np.sqrt(2.0 * d)
    c = datagen.c6_moe_drelu_ffn(rows, d=d, ffn=ffn, n_experts=e, bias=-0.2864 * sigma)
    note(f"moe det={det} rows={rows} d={d} ffn={ffn} E={e} k={k}")
    with reduction_mode(gpu_lib, det):
        zf = _moe_case(gpu_lib, c, k)
    assert 0.6 < zf < 0.98


@pytest.mark.parametrize("det", [False, True])
def test_moe_bf16_output(gpu_lib, det):
    import torch
    c = datagen.c6_moe_drelu_ffn(2, d=256, ffn=512, bias=-0.13)
    note(f"moe bf16 y det={det}")
    with reduction_mode(gpu_lib, det):
        _moe_case(gpu_lib, c, 2, ydt=torch.bfloat16)


def test_moe_full_mixtral(gpu_lib):
    """Mixtral-47B-shaped layer: d = 4096, ffn = 14336, 8 experts, top-2, biases
    set for ~85% inactive neurons per expert (the summary's figure); batches
    of 1 and 4 tokens on the same weights."""
    c = datagen.c6_moe_drelu_ffn(1)
    for batch in (1, 4):
        if batch != 1:
            c["X"] = datagen.c6_moe_drelu_ffn(batch, with_weights=False)["X"]
        note(f"moe full Mixtral shape batch={batch}")
        zf = _moe_case(gpu_lib, c, 2)
        assert 0.80 < zf < 0.90
