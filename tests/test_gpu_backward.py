"""GPU parity of the sparse-activation linear's backward with the
straight-through estimator (qs_sparse_linear_backward):
dX = dY . W (not masked) and dW = dY^T . (X (.) M).

Tolerance: the products of bf16 inputs are exact in fp32 and the sums are
fp32 on matrix cores, so |g - g_ref| <= 4e-3 * T with T the sum of the
absolute products (T_dx = |dY| . |W|, T_dw = |dY|^T . |X (.) M|), the same
budget as the bf16 forward, which also covers a bf16 output's rounding.
T == 0 (a feature column no row selected) requires an exact zero.
Integer-valued inputs make every partial sum exact: bit-exact there.
"""
import numpy as np
import pytest

import datagen
import oracle
from gpu_util import assert_within, note, to_dev

pytestmark = pytest.mark.gpu


def _case(seed, rows, d, n):
    rng = np.random.default_rng(seed)
    x = datagen.bf16_round(datagen.student_t(rng, (rows, d)))
    w = datagen.bf16_round(datagen.normal(rng, (n, d), 0.02))
    gy = datagen.bf16_round(datagen.normal(rng, (rows, n), 1.0))
    return x, w, gy


def _run(qs, x, k, w, gy, layout, out_dtype):
    import torch
    xd = to_dev(x, torch.bfloat16)
    wd = to_dev(np.ascontiguousarray(w.T) if layout == qs.LAYOUT_WT else w, torch.bfloat16)
    gd = to_dev(gy, torch.bfloat16)
    dx, dw = qs.qs_sparse_linear_backward(xd, k, wd, gd, layout=layout, out_dtype=out_dtype)
    torch.cuda.synchronize()
    dw = dw.float().cpu().numpy()
    if layout == qs.LAYOUT_WT:
        dw = dw.T
    return dx.float().cpu().numpy(), dw


def _ref(x, k, w, gy):
    mask, _, _, _ = oracle.topk_select(oracle.magnitude(x), k)
    return oracle.sparse_linear_backward(x, w, mask, gy)


@pytest.mark.parametrize("layout", ["W", "WT"])
@pytest.mark.parametrize("rows,d,n", [(1, 64, 40), (5, 64, 48), (37, 200, 304),
                                      (300, 520, 200), (513, 128, 776), (64, 1024, 264)])
def test_backward_random(gpu_lib, layout, rows, d, n):
    import torch
    qs = gpu_lib
    lay = qs.LAYOUT_W if layout == "W" else qs.LAYOUT_WT
    x, w, gy = _case(rows * 5 + d + n, rows, d, n)
    for k in sorted({0, 1, (7 * d) // 10, d}):
        note(f"backward layout={layout} rows={rows} d={d} n={n} k={k}")
        dx, dw = _run(qs, x, k, w, gy, lay, torch.float32)
        ref = _ref(x, k, w, gy)
        assert_within(dx, ref["dx"], ref["T_dx"], 4e-3, f"dx k={k}")
        assert_within(dw, ref["dw"], ref["T_dw"], 4e-3, f"dw k={k}")


@pytest.mark.parametrize("layout", ["W", "WT"])
def test_backward_integer_valued_is_exact(gpu_lib, layout):
    import torch
    qs = gpu_lib
    lay = qs.LAYOUT_W if layout == "W" else qs.LAYOUT_WT
    rng = np.random.default_rng(71)
    rows, d, n = 300, 264, 392
    x = rng.integers(-8, 9, size=(rows, d)).astype(np.float32)
    w = rng.integers(-2, 3, size=(n, d)).astype(np.float32)
    gy = rng.integers(-4, 5, size=(rows, n)).astype(np.float32)
    note(f"backward integer-valued layout={layout}")
    dx, dw = _run(qs, x, 100, w, gy, lay, torch.float32)
    ref = _ref(x, 100, w, gy)
    assert np.array_equal(dx, ref["dx"])
    assert np.array_equal(dw, ref["dw"])


def test_backward_bf16_outputs_and_single_gradients(gpu_lib):
    import torch
    qs = gpu_lib
    x, w, gy = _case(5, 70, 256, 136)
    k = 100
    ref = _ref(x, k, w, gy)
    note("backward bf16 outputs")
    dx, dw = _run(qs, x, k, w, gy, qs.LAYOUT_W, torch.bfloat16)
    assert_within(dx, ref["dx"], ref["T_dx"], 4e-3, "dx bf16")
    assert_within(dw, ref["dw"], ref["T_dw"], 4e-3, "dw bf16")
    xd, wd, gd = to_dev(x, torch.bfloat16), to_dev(w, torch.bfloat16), to_dev(gy, torch.bfloat16)
    note("backward dx only / dw only")
    dx1, dw1 = qs.qs_sparse_linear_backward(xd, k, wd, gd, layout=qs.LAYOUT_W, want_dw=False)
    dx2, dw2 = qs.qs_sparse_linear_backward(xd, k, wd, gd, layout=qs.LAYOUT_W, want_dx=False)
    full_dx, full_dw = qs.qs_sparse_linear_backward(xd, k, wd, gd, layout=qs.LAYOUT_W)
    torch.cuda.synchronize()
    assert dw1 is None and dx2 is None
    assert torch.equal(dx1, full_dx) and torch.equal(dw2, full_dw)


def test_backward_empty_batch_gives_zero_weight_gradient(gpu_lib):
    import torch
    qs = gpu_lib
    d, n = 64, 48
    x = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    gy = torch.empty((0, n), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((n, d), dtype=torch.bfloat16, device="cuda")
    dw = torch.full((n, d), 7.0, dtype=torch.float32, device="cuda")
    note("backward rows=0")
    dx, dw = qs.qs_sparse_linear_backward(x, 10, w, gy, layout=qs.LAYOUT_W, dw=dw)
    torch.cuda.synchronize()
    assert dx.shape == (0, d)
    assert int(dw.count_nonzero()) == 0


def test_backward_deterministic(gpu_lib):
    import torch
    qs = gpu_lib
    x, w, gy = _case(9, 300, 512, 384)
    xd, wd, gd = to_dev(x, torch.bfloat16), to_dev(w, torch.bfloat16), to_dev(gy, torch.bfloat16)
    note("backward determinism")
    a = qs.qs_sparse_linear_backward(xd, 200, wd, gd, layout=qs.LAYOUT_W)
    b = qs.qs_sparse_linear_backward(xd, 200, wd, gd, layout=qs.LAYOUT_W)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("layout", ["W", "WT"])
def test_backward_full_c4_sampled(gpu_lib, layout):
    """The fused-QKV shape as a training step: X [2048, 4096], W [12288, 4096],
    K = 2867, dY [2048, 12288].  The oracle checks sampled rows of dX (all
    4096 entries each) and sampled output neurons of dW (all 4096 input
    features each), covering every tile of both GEMMs, at the launch shapes
    the bench times."""
    import torch
    qs = gpu_lib
    lay = qs.LAYOUT_W if layout == "W" else qs.LAYOUT_WT
    c = datagen.c4_prefill_qkv()
    x, w, k = c["X"], c["W"], c["K"]
    gy = datagen.c4_backward_grad(x.shape[0], w.shape[0])
    note(f"backward full C4 layout={layout}")
    dx, dw = _run(qs, x, k, w, gy, lay, torch.float32)
    rng = np.random.default_rng(73)
    # One sampled token in every 256-token block (the dX GEMM's M tiles) and
    # one output neuron in every 128-neuron block, which meets every M tile of
    # the W-layout dW GEMM (256 neurons) and every N tile (128 or 192
    # neurons) of the W^T-layout one; every checked row or neuron is checked
    # over all 4096 features, i.e. across every tile of the other dimension.
    rows = np.array([b + rng.integers(0, 256) for b in range(0, x.shape[0], 256)])
    outs = np.array([b + rng.integers(0, 128) for b in range(0, w.shape[0], 128)])
    rows = np.unique(np.concatenate([rows, [0, x.shape[0] - 1]]))
    outs = np.unique(np.concatenate([outs, [0, w.shape[0] - 1]]))
    mask, _, _, _ = oracle.topk_select(oracle.magnitude(x), k)
    r_dx = oracle.sparse_linear_backward(x[rows], w, mask[rows], gy[rows])
    assert_within(dx[rows], r_dx["dx"], r_dx["T_dx"], 4e-3, "C4 dx")
    # dW rows o: dY[:, o]^T . (X (.) M) over all tokens, with W restricted to those outputs
    r_dw = oracle.sparse_linear_backward(x, w[outs], mask, gy[:, outs])
    assert_within(dw[outs], r_dw["dw"], r_dw["T_dw"], 4e-3, "C4 dw")
