"""Canary bands: every output buffer and the workspace of each entry point is
placed between guard regions of a known byte pattern, at ragged shapes (rows,
features and columns that fill no tile, stage or wavefront evenly), through
each internal path (one-token column kernel, gathers, matrix-core paths, the
fixed-order and the atomic sums).  After the call every guard byte must be
intact: no kernel writes past the end (or before the start) of a buffer
include/qs.h gives it.
"""
import numpy as np
import pytest

import datagen
from gpu_util import note, reduction_mode, to_dev

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes on each side (keeps 256-byte alignment)
PATTERN = 0xA5


class Guarded:
    """A device tensor of `shape`/`dtype` in the middle of a guarded buffer."""

    def __init__(self, shape, dtype, nbytes=None):
        import torch
        itemsize = torch.empty((), dtype=dtype).element_size()
        self.n = int(np.prod(shape)) * itemsize if nbytes is None else nbytes
        self.buf = torch.full((GUARD + self.n + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        body = self.buf[GUARD:GUARD + self.n]
        self.t = body.view(dtype).view(shape) if nbytes is None else body

    def intact(self):
        b = self.buf.cpu().numpy()
        return bool(np.all(b[:GUARD] == PATTERN) and np.all(b[GUARD + self.n:] == PATTERN))


def _ws(qs, op, rows, d, n):
    import torch
    return Guarded((max(qs.qs_workspace_bytes(op, rows, d, n), 1),), torch.uint8,
                   nbytes=max(qs.qs_workspace_bytes(op, rows, d, n), 1))


def _check(what, *guards):
    import torch
    torch.cuda.synchronize()
    for i, g in enumerate(guards):
        assert g.intact(), f"{what}: guard band of buffer {i} overwritten"


@pytest.mark.parametrize("kind", ["f32", "bf16", "i8"])
def test_canary_topk(gpu_lib, kind):
    import torch
    qs = gpu_lib
    rows, d, k = 3, 1001 if kind != "bf16" else 1002, 400
    rng = np.random.default_rng(5)
    x = datagen.student_t(rng, (rows, d))
    xd = (to_dev(x) if kind == "f32" else to_dev(x, torch.bfloat16) if kind == "bf16"
          else to_dev(np.clip(np.round(x * 20), -128, 127).astype(np.int8)))
    mask, idx = Guarded((rows, d), torch.uint8), Guarded((rows, k), torch.int32)
    tau, cut = Guarded((rows,), torch.int32), Guarded((rows,), torch.int32)
    xs = Guarded((rows, d), torch.float32) if kind != "i8" else None   # (no xs for int8 x)
    note(f"canary topk {kind}")
    qs.qs_topk_mask(xd, k, mask=mask.t, idx=idx.t, tau=tau.t, cutoff=cut.t,
                    xs=xs.t if xs else None)
    _check("topk", *[g for g in (mask, idx, tau, cut, xs) if g is not None])


@pytest.mark.parametrize("det", [False, True])
@pytest.mark.parametrize("rows,d,n,wt,layout", [
    (1, 1000, 520, "bf16", "WT"),      # one bf16 token: the column kernel
    (3, 1000, 520, "bf16", "WT"),      # gather
    (12, 700, 264, "bf16", "WT"),      # 16-token matrix-core gather, ragged tile
    (5, 700, 260, "f32", "WT"),        # fp32 gather
    (37, 264, 136, "bf16", "W"),       # masked dense MFMA
])
def test_canary_linear(gpu_lib, det, rows, d, n, wt, layout):
    import torch
    qs = gpu_lib
    dt = torch.bfloat16 if wt == "bf16" else torch.float32
    rng = np.random.default_rng(rows + d + n)
    x = datagen.student_t(rng, (rows, d))
    w = datagen.normal(rng, (n, d), 0.02)
    lay = qs.LAYOUT_WT if layout == "WT" else qs.LAYOUT_W
    wd = to_dev(np.ascontiguousarray(w.T) if layout == "WT" else w, dt)
    for ydt in (torch.float32, torch.bfloat16):
        y = Guarded((rows, n), ydt)
        ws = _ws(qs, qs.OP_SPARSE_LINEAR, rows, d, n)
        note(f"canary linear det={det} {rows}x{d}x{n} {wt} {layout} y={ydt}")
        with reduction_mode(qs, det):
            qs.qs_sparse_linear(to_dev(x, dt), (2 * d) // 5, wd, layout=lay, y=y.t, ws=ws.t)
        _check("linear", y, ws)


def test_canary_gathers(gpu_lib):
    import torch
    qs = gpu_lib
    rng = np.random.default_rng(9)
    rows, d, n = 5, 700, 264
    xs = datagen.student_t(rng, (rows, d)) * (rng.random((rows, d)) < 0.4)
    wt = to_dev(np.ascontiguousarray(datagen.normal(rng, (n, d), 0.02).T), torch.bfloat16)
    ws = Guarded((1,), torch.uint8, nbytes=qs.qs_workspace_bytes(qs.OP_GATHER_LINEAR, rows, d, n))
    ws.t.zero_()
    y = Guarded((rows, n), torch.float32)
    note("canary gather_linear / _acc")
    qs.qs_gather_linear(to_dev(xs), wt, y=y.t, ws=ws.t)
    qs.qs_gather_linear_acc(to_dev(xs), wt, y.t, ws=ws.t)
    _check("gather", y, ws)
    x = datagen.student_t(rng, (2, 1004))
    wt2 = to_dev(np.ascontiguousarray(datagen.normal(rng, (520, 1004), 0.02).T), torch.bfloat16)
    y2 = Guarded((2, 520), torch.float32)
    y2.t.zero_()
    note("canary topk_gather_linear_acc")
    qs.qs_topk_gather_linear_acc(to_dev(x), 401, wt2, y2.t)
    _check("topk gather acc", y2)


@pytest.mark.parametrize("rows", [1, 3, 17])
def test_canary_i8t(gpu_lib, rows):
    import torch
    qs = gpu_lib
    rng = np.random.default_rng(rows)
    d, n, k = 1000, 1040, 388
    x = datagen.student_t(rng, (rows, d))
    t = qs.qs_ternarize(datagen.normal(rng, (n, d), 0.02))
    wp = to_dev(qs.qs_pack_ternary(t[0]))
    acc, y = Guarded((rows, n), torch.int32), Guarded((rows, n), torch.float32)
    xq, xsc = Guarded((rows, d), torch.int8), Guarded((rows,), torch.float32)
    idx = Guarded((rows, k), torch.int32)
    ws = _ws(qs, qs.OP_SPARSE_LINEAR_I8T, rows, d, n)
    note(f"canary i8t rows={rows}")
    qs.qs_sparse_linear_i8t(to_dev(x), k, wp, float(t[1]), n, acc=acc.t, y=y.t, xq=xq.t,
                            xscale=xsc.t, idx=idx.t, ws=ws.t)
    _check("i8t", acc, y, xq, xsc, idx, ws)


@pytest.mark.parametrize("det", [False, True])
@pytest.mark.parametrize("act,rows,d,f", [
    ("relu2", 1, 256, 520), ("relu2", 3, 256, 520), ("relu2", 17, 512, 264),
    ("glu", 1, 128, 200), ("glu", 2, 128, 200), ("drelu", 4, 200, 136), ("drelu", 1, 64, 48),
])
def test_canary_ffn(gpu_lib, det, act, rows, d, f):
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    rng = np.random.default_rng(rows * 3 + d + f)
    x = datagen.bf16_round(datagen.student_t(rng, (rows, d)))
    wu = to_dev(datagen.normal(rng, (f, d), 0.02), bf)
    wd = to_dev(np.ascontiguousarray(datagen.normal(rng, (d, f), 0.02).T), bf)
    kw = {}
    a = {"relu2": qs.ACT_RELU2, "glu": qs.ACT_RELU2_GLU, "drelu": qs.ACT_DRELU}[act]
    k_in, k_mid = (2 * d) // 5, (2 * f) // 5
    if act == "glu":
        kw["w_gate"] = to_dev(np.ascontiguousarray(datagen.normal(rng, (f, d), 0.02).T), bf)
        wu = to_dev(np.ascontiguousarray(datagen.normal(rng, (f, d), 0.02).T), bf)
    elif act == "relu2":
        wu = to_dev(np.ascontiguousarray(datagen.normal(rng, (f, d), 0.02).T), bf)
    else:
        kw["w_gate"] = to_dev(datagen.normal(rng, (f, d), 0.02), bf)
        kw["b_gate"] = to_dev(np.full(f, -0.02, np.float32))
        kw["b_up"] = to_dev(np.zeros(f, np.float32))
        k_in, k_mid = d, -1
    op = {"relu2": qs.OP_SPARSE_FFN_RELU2, "glu": qs.OP_SPARSE_FFN_RELU2_GLU,
          "drelu": qs.OP_SPARSE_FFN_DRELU}[act]
    for outputs in (False, True):
        y = Guarded((rows, d), torch.float32)
        h = Guarded((rows, f), torch.float32) if outputs else None
        mi = Guarded((rows, f), torch.int32) if outputs else None
        mc = Guarded((rows,), torch.int32) if outputs else None
        ws = _ws(qs, op, rows, d, f)
        note(f"canary ffn {act} det={det} rows={rows} d={d} f={f} outputs={outputs}")
        with reduction_mode(qs, det):
            qs.qs_sparse_ffn(to_dev(x, bf), a, k_in, k_mid, wu, wd, y=y.t,
                             h=h.t if h else None, mid_idx=mi.t if mi else None,
                             mid_cnt=mc.t if mc else None, ws=ws.t, **kw)
        _check("ffn", *[g for g in (y, h, mi, mc, ws) if g is not None])


def test_canary_backward_block_moe(gpu_lib):
    import torch
    qs = gpu_lib
    bf = torch.bfloat16
    rng = np.random.default_rng(77)
    rows, d, n = 40, 264, 136
    x = to_dev(datagen.student_t(rng, (rows, d)), bf)
    w = to_dev(datagen.normal(rng, (n, d), 0.02), bf)
    dy = to_dev(datagen.normal(rng, (rows, n), 1.0), bf)
    dx, dw = Guarded((rows, d), torch.float32), Guarded((n, d), torch.float32)
    ws = _ws(qs, qs.OP_SPARSE_LINEAR_BACKWARD, rows, d, n)
    note("canary backward")
    qs.qs_sparse_linear_backward(x, 100, w, dy, dx=dx.t, dw=dw.t, ws=ws.t)
    _check("backward", dx, dw, ws)
    db = 288   # (the 2:4 path takes d_in % 32 == 0)
    xb = to_dev(datagen.student_t(rng, (rows, db)), bf)
    wb = to_dev(datagen.normal(rng, (n, db), 0.02), bf)
    y, m = Guarded((rows, n), torch.float32), Guarded((rows, db), torch.uint8)
    ws = _ws(qs, qs.OP_BLOCK_SPARSE_LINEAR, rows, db, n)
    note("canary block 2:4")
    qs.qs_block_sparse_linear(xb, wb, y=y.t, want_mask=True, mask=m.t, ws=ws.t)
    _check("block", y, m, ws)
    e, f, top = 4, 72, 2
    xm = to_dev(datagen.bf16_round(datagen.student_t(rng, (3, d))), bf)
    wr = to_dev(datagen.normal(rng, (e, d), 0.02), bf)
    wg, wu, wdn = (to_dev(datagen.normal(rng, (e, f, d), 0.02), bf) for _ in range(3))
    bg = to_dev(np.full((e, f), -0.01, np.float32))
    bu = to_dev(np.zeros((e, f), np.float32))
    y = Guarded((3, d), torch.float32)
    ws = _ws(qs, qs.OP_SPARSE_MOE_FFN, 3 * top, d, f)
    note("canary moe")
    qs.qs_sparse_moe_ffn(xm, top, wr, wg, wu, wdn, b_gate=bg, b_up=bu, y=y.t, ws=ws.t)
    _check("moe", y, ws)
