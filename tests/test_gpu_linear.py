"""GPU parity of the sparse-activation linear Y = (X (.) M) . W^T.

Tolerances (fp32 accumulation of exact products): |y - y_ref| <= 1e-5 * T for
fp32 inputs and <= 4e-3 * T for bf16 inputs (which also covers a bf16 output
rounding), T = sum over selected j of |x_j w_j|; T == 0 requires y == 0.
Integer-valued inputs make every partial sum exact, so there the result must
be bit-exact whatever the reduction order.
"""
import numpy as np
import pytest

import datagen
import oracle
from gpu_util import assert_within, note, reduction_mode, to_dev

pytestmark = pytest.mark.gpu


def _run(gpu_lib, x, k, w, xdt, wdt, ydt, layout=None):
    import torch
    qs = gpu_lib
    layout = qs.LAYOUT_WT if layout is None else layout
    xd = to_dev(x, xdt)
    wd = to_dev(np.ascontiguousarray(w.T) if layout == qs.LAYOUT_WT else w, wdt)
    y = qs.qs_sparse_linear(xd, k, wd, layout=layout, y_dtype=ydt)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


def _ref(x, k, w):
    mask, _, _, _ = oracle.topk_select(oracle.magnitude(x), k)
    return oracle.sparse_linear(x, w, mask)


@pytest.mark.parametrize("wtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,d,n", [(1, 64, 8), (3, 300, 264), (8, 1024, 1024),
                                      (20, 700, 520), (37, 256, 128), (1, 4096, 11008)])
def test_linear_random(gpu_lib, wtype, rows, d, n):
    import torch
    rng = np.random.default_rng(rows * 7 + d + n)
    x = datagen.student_t(rng, (rows, d))
    w = datagen.normal(rng, (n, d), 0.02)
    dt = torch.float32 if wtype == "f32" else torch.bfloat16
    if wtype == "bf16":
        x, w = datagen.bf16_round(x), datagen.bf16_round(w)
    tol = 1e-5 if wtype == "f32" else 4e-3
    for k in sorted({0, 1, (2 * d) // 5, d}):
        note(f"linear {wtype} rows={rows} d={d} n={n} k={k}")
        y = _run(gpu_lib, x, k, w, dt, dt, torch.float32)
        y_ref, t = _ref(x, k, w)
        assert_within(y, y_ref, t, tol, f"linear {wtype} k={k}")


@pytest.mark.parametrize("d,n", [(8, 8), (1000, 1040), (8192, 520), (256, 16384), (4096, 11008)])
def test_linear_one_bf16_token(gpu_lib, d, n):
    """One bf16 token, bf16 W^T: the single-launch column kernel (selection
    inside every workgroup, fixed-order sums), fp32 and bf16 y; two calls in
    the default (atomic) reduction mode agree bitwise."""
    import torch
    rng = np.random.default_rng(d + 3 * n)
    x = datagen.bf16_round(datagen.student_t(rng, (1, d)))
    w = datagen.bf16_round(datagen.normal(rng, (n, d), 0.02))
    for k in sorted({0, 1, 7, (2 * d) // 5, d - 1, d}):
        note(f"linear one bf16 token d={d} n={n} k={k}")
        y = _run(gpu_lib, x, k, w, torch.bfloat16, torch.bfloat16, torch.float32)
        y2 = _run(gpu_lib, x, k, w, torch.bfloat16, torch.bfloat16, torch.float32)
        assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
        y_ref, t = _ref(x, k, w)
        assert_within(y, y_ref, t, 4e-3, f"one token k={k}")
        yb = _run(gpu_lib, x, k, w, torch.bfloat16, torch.bfloat16, torch.bfloat16)
        # bf16 output: the fp32 result rounded to nearest-even
        exp = torch.from_numpy(y).to(torch.bfloat16).float().numpy()
        assert np.array_equal(yb, exp), "bf16 y is not the rounded fp32 y"


@pytest.mark.parametrize("wtype", ["f32", "bf16"])
def test_linear_integer_valued_is_exact(gpu_lib, wtype):
    import torch
    rng = np.random.default_rng(41)
    rows, d, n = 6, 2000, 776
    x = rng.integers(-30, 31, size=(rows, d)).astype(np.float32)
    w = rng.integers(-3, 4, size=(n, d)).astype(np.float32)
    dt = torch.float32 if wtype == "f32" else torch.bfloat16
    note(f"linear integer-valued {wtype}")
    y = _run(gpu_lib, x, 900, w, dt, dt, torch.float32)
    y_ref, _ = _ref(x, 900, w)
    assert np.array_equal(y, y_ref)


def test_linear_bf16_output_and_dense_k(gpu_lib):
    import torch
    rng = np.random.default_rng(43)
    x = datagen.bf16_round(datagen.student_t(rng, (4, 512)))
    w = datagen.bf16_round(datagen.normal(rng, (256, 512), 0.02))
    note("linear bf16 output, k = d")
    y = _run(gpu_lib, x, 512, w, torch.bfloat16, torch.bfloat16, torch.bfloat16)
    y_ref = x.astype(np.float64) @ w.astype(np.float64).T       # K = D: the dense product
    t = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    assert_within(y, y_ref, t, 4e-3, "bf16 out")


def test_linear_deterministic(gpu_lib):
    """With fixed-order sums two runs agree bit for bit; the default (atomic)
    sums stay within the same tolerance of the oracle in every run."""
    import torch
    rng = np.random.default_rng(47)
    x = datagen.bf16_round(datagen.student_t(rng, (5, 4096)))
    w = datagen.bf16_round(datagen.normal(rng, (4096, 4096), 0.02))
    note("linear run-twice determinism")
    with reduction_mode(gpu_lib, True):
        y1 = _run(gpu_lib, x, 1638, w, torch.bfloat16, torch.bfloat16, torch.float32)
        y2 = _run(gpu_lib, x, 1638, w, torch.bfloat16, torch.bfloat16, torch.float32)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    y_ref, t = _ref(x, 1638, w)
    assert_within(y1, y_ref, t, 4e-3, "fixed order")
    note("linear atomic split-K sums")
    with reduction_mode(gpu_lib, False):
        for _ in range(2):
            y3 = _run(gpu_lib, x, 1638, w, torch.bfloat16, torch.bfloat16, torch.float32)
            assert_within(y3, y_ref, t, 4e-3, "atomic sums")


@pytest.mark.parametrize("wtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,d,n", [(1, 4096, 1024), (3, 1000, 520), (8, 2048, 264),
                                      (16, 4096, 1024)])
def test_gather_linear_acc(gpu_lib, wtype, rows, d, n):
    """qs_gather_linear_acc adds Xs . W^T to what y holds (every kernel form:
    1-8 token tiles, and 16-token bf16 MFMA tiles); fp32 weights in 16-token
    tiles are refused."""
    import torch
    qs = gpu_lib
    rng = np.random.default_rng(rows * 7 + d + n)
    x = datagen.student_t(rng, (rows, d))
    w = datagen.normal(rng, (n, d), 0.02)
    y0 = datagen.normal(rng, (rows, n), 1.0).astype(np.float32)
    dt = torch.float32 if wtype == "f32" else torch.bfloat16
    tol = 1e-5 if wtype == "f32" else 4e-3
    if wtype == "bf16":
        x, w = datagen.bf16_round(x), datagen.bf16_round(w)
    k = (2 * d) // 5
    m_ref, _, _, _ = oracle.topk_select(oracle.magnitude(x), k)
    xs = np.where(m_ref == 1, x, 0.0).astype(np.float32)
    wt = to_dev(np.ascontiguousarray(w.T), dt)
    y = to_dev(y0)
    note(f"gather_linear_acc {wtype} rows={rows} d={d} n={n}")
    if wtype == "f32" and rows > 8:
        with pytest.raises(qs.QSError):
            qs.qs_gather_linear_acc(to_dev(xs), wt, y)
        return
    qs.qs_gather_linear_acc(to_dev(xs), wt, y)
    torch.cuda.synchronize()
    y_ref, t = oracle.sparse_linear(x, w, m_ref)
    got = y.cpu().numpy().astype(np.float64) - y0
    # Each of the (at most 64) split additions into y0 rounds once in fp32 on a
    # value of magnitude <= |y0| + T.
    slack = 64 * 2.0 ** -24 * (np.abs(y0.astype(np.float64)) + t)
    assert np.all(np.abs(got - y_ref) <= tol * t + slack), "y - y0 outside tol*T"


def test_linear_full_c1(gpu_lib):
    import torch
    c = datagen.c1_linear()
    note("linear full config C1 fp32 [8,1024] x [1024,1024], K=410")
    y = _run(gpu_lib, c["X"], c["K"], c["W"], torch.float32, torch.float32, torch.float32)
    y_ref, t = _ref(c["X"], c["K"], c["W"])
    assert_within(y, y_ref, t, 1e-5, "C1")


@pytest.mark.parametrize("batch", [1, 2, 4, 8, 16])
def test_linear_full_c2_up(gpu_lib, batch):
    """The Llama-7B FFN up projection at decode batch sizes (bf16, K = 1638)."""
    import torch
    c = datagen.c2_relu2_ffn(batch)
    note(f"linear C2 up projection B={batch}")
    y = _run(gpu_lib, c["X"], c["K_in"], c["W_up"], torch.bfloat16, torch.bfloat16, torch.float32)
    y_ref, t = _ref(c["X"], c["K_in"], c["W_up"])
    assert_within(y, y_ref, t, 4e-3, f"C2 up B={batch}")


def test_topk_xs_and_gather_linear(gpu_lib):
    """qs_topk_mask's xs output is X (.) M, and qs_gather_linear on it gives the
    same product (workspace reused across calls, counters left zero)."""
    import torch
    qs = gpu_lib
    rng = np.random.default_rng(59)
    ws = None
    for rows, d, n, k in [(3, 1000, 520, 400), (16, 4096, 1024, 1638), (1, 300, 64, 7)]:
        x = datagen.bf16_round(datagen.student_t(rng, (rows, d)))
        w = datagen.bf16_round(datagen.normal(rng, (n, d), 0.02))
        note(f"gather_linear rows={rows} d={d} n={n} k={k}")
        mask, _, _, _, xs = qs.qs_topk_mask(to_dev(x, torch.bfloat16), k, want_xs=True)
        if ws is None or ws.numel() < qs.qs_workspace_bytes(qs.OP_GATHER_LINEAR, rows, d, n):
            ws = qs.gather_workspace(16, 4096, 1024)
        y = qs.qs_gather_linear(xs, to_dev(np.ascontiguousarray(w.T), torch.bfloat16), ws=ws)
        torch.cuda.synchronize()
        m_ref, _, _, _ = oracle.topk_select(oracle.magnitude(x), k)
        assert np.array_equal(xs.cpu().numpy(), np.where(m_ref == 1, x, 0.0).astype(np.float32))
        y_ref, t = oracle.sparse_linear(x, w, m_ref)
        assert_within(y.cpu().numpy(), y_ref, t, 4e-3, "gather_linear")
        assert int(ws[:16384].count_nonzero()) == 0, "split-K counters must be left zero"


# ---------------------------------------------------------------- MFMA (batched) path

@pytest.mark.parametrize("rows,d,n", [(1, 64, 40), (37, 200, 300), (256, 512, 256),
                                      (300, 1000, 520), (513, 128, 777)])
def test_linear_mfma_random(gpu_lib, rows, d, n):
    import torch
    qs = gpu_lib
    rng = np.random.default_rng(rows + 3 * d + n)
    x = datagen.bf16_round(datagen.student_t(rng, (rows, d)))
    w = datagen.bf16_round(datagen.normal(rng, (n, d), 0.02))
    for k in sorted({0, 1, (7 * d) // 10, d}):
        note(f"linear MFMA rows={rows} d={d} n={n} k={k}")
        y = _run(gpu_lib, x, k, w, torch.bfloat16, torch.bfloat16, torch.float32,
                 layout=qs.LAYOUT_W)
        y_ref, t = _ref(x, k, w)
        assert_within(y, y_ref, t, 4e-3, f"mfma k={k}")


@pytest.mark.parametrize("rows,d,n,k", [(300, 512, 400, 300), (100, 4096, 264, 2867),
                                        (97, 2056, 136, 1)])
def test_linear_mfma_integer_valued_is_exact(gpu_lib, rows, d, n, k):
    """Integer-valued x (|x| <= 8: most of the selection is decided by the
    index rule among equal magnitudes) and w: y is exact, so it is equal to
    the oracle's only if the selection (run for many rows by the two-level
    bf16 selection kernel) is the oracle's."""
    import torch
    qs = gpu_lib
    rng = np.random.default_rng(61 + d)
    x = rng.integers(-8, 9, size=(rows, d)).astype(np.float32)
    w = rng.integers(-2, 3, size=(n, d)).astype(np.float32)
    note(f"linear MFMA integer-valued rows={rows} d={d} k={k}")
    y = _run(gpu_lib, x, k, w, torch.bfloat16, torch.bfloat16, torch.float32, layout=qs.LAYOUT_W)
    y_ref, _ = _ref(x, k, w)
    assert np.array_equal(y, y_ref)


def test_linear_mfma_full_c4_sampled(gpu_lib):
    """Fused-QKV prefill: X [2048,4096] bf16, W [12288,4096], K = 2867; the
    oracle checks 96 sampled rows (all 12288 outputs each) and the output is
    also produced in bf16."""
    import torch
    qs = gpu_lib
    c = datagen.c4_prefill_qkv()
    x, w, k = c["X"], c["W"], c["K"]
    note("linear MFMA full config C4")
    y = _run(gpu_lib, x, k, w, torch.bfloat16, torch.bfloat16, torch.float32, layout=qs.LAYOUT_W)
    yb = _run(gpu_lib, x, k, w, torch.bfloat16, torch.bfloat16, torch.bfloat16, layout=qs.LAYOUT_W)
    rows = np.sort(np.random.default_rng(67).choice(x.shape[0], 96, replace=False))
    rows[0], rows[-1] = 0, x.shape[0] - 1
    y_ref, t = _ref(x[rows], k, w)
    assert_within(y[rows], y_ref, t, 4e-3, "C4 fp32 out")
    assert_within(yb[rows], y_ref, t, 4e-3, "C4 bf16 out")


@pytest.mark.parametrize("rows", [5, 8, 16, 23])
@pytest.mark.parametrize("det", [False, True])
def test_linear_fp32_x_bf16_w(gpu_lib, rows, det):
    """fp32 activations with bf16 weights: tiles of 8-16 tokens run the bf16
    matrix-core gather, which carries each fp32 coefficient as a two-term
    bf16 split (relative error at most 2^-18); with fp32 accumulation the
    result stays within the fp32 bound 1e-5 * T."""
    import torch
    rng = np.random.default_rng(500 + rows)
    d, n = 1536, 1032
    x = datagen.student_t(rng, (rows, d))
    w = datagen.bf16_round(datagen.normal(rng, (n, d), 0.02))
    with reduction_mode(gpu_lib, det):
        for k in (d // 3, d):
            note(f"linear fp32 x / bf16 w rows={rows} k={k} det={det}")
            y = _run(gpu_lib, x, k, w, torch.float32, torch.bfloat16, torch.float32)
            y_ref, t = _ref(x, k, w)
            assert_within(y, y_ref, t, 1e-5, f"fp32 x, bf16 w, rows={rows}")
