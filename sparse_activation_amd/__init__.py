"""Python binding of libqs.so, the MI355X (gfx950) Q-Sparse hot path.

Thin ctypes wrappers with the names of the C entry points in include/qs.h.
They only marshal arguments: check dtypes, shapes and devices of torch
tensors, allocate outputs and workspaces with torch when the caller passes
none, and pass raw device pointers and the current HIP stream to the
library.  All computation runs in the library's HIP kernels; there is no
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "load", "lib_path", "QS_OK", "QSError",
    "qs_topk_mask", "qs_gather_linear", "gather_workspace", "qs_sparse_linear",
    "qs_sparse_linear_i8t", "qs_sparse_ffn",
    "qs_workspace_bytes", "qs_ternarize", "qs_pack_ternary", "qs_last_error", "qs_version",
    "F32", "BF16", "I8", "LAYOUT_WT", "LAYOUT_W", "ACT_RELU2", "ACT_DRELU", "ACT_RELU2_GLU",
    "OP_TOPK_MASK", "OP_SPARSE_LINEAR", "OP_SPARSE_LINEAR_I8T", "OP_SPARSE_FFN_RELU2",
    "OP_SPARSE_FFN_DRELU", "OP_GATHER_LINEAR", "OP_SPARSE_FFN_RELU2_GLU",
    "OP_SPARSE_LINEAR_BACKWARD", "qs_sparse_linear_backward", "OP_BLOCK_SPARSE_LINEAR",
    "qs_block_sparse_linear", "OP_SPARSE_MOE_FFN", "qs_sparse_moe_ffn",
    "qs_gather_linear_acc", "qs_topk_gather_linear_acc", "qs_set_deterministic",
    "qs_sparse_ffn_static", "qs_sparse_linear_pitched", "qs_sparse_ffn_pitched",
    "STATIC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))

QS_OK, QS_ERR_INVALID_ARG, QS_ERR_UNSUPPORTED, QS_ERR_WORKSPACE, QS_ERR_HIP = range(5)
STATIC_SCRATCH_BYTES = 32 << 20   # QS_STATIC_SCRATCH_BYTES
F32, BF16, I8 = 0, 1, 2
LAYOUT_WT, LAYOUT_W = 0, 1
ACT_RELU2, ACT_DRELU, ACT_RELU2_GLU = 0, 1, 2
(OP_TOPK_MASK, OP_SPARSE_LINEAR, OP_SPARSE_LINEAR_I8T, OP_SPARSE_FFN_RELU2,
 OP_SPARSE_FFN_DRELU, OP_GATHER_LINEAR, OP_SPARSE_FFN_RELU2_GLU,
 OP_SPARSE_LINEAR_BACKWARD, OP_BLOCK_SPARSE_LINEAR, OP_SPARSE_MOE_FFN) = range(10)

# Every function the header declares, with its ctypes signature.
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SIGS = {
    "qs_topk_mask": [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P],
    "qs_gather_linear": [_P, _I64, _I64, _P, _INT, _I64, _I64, _P, _INT, _P, ctypes.c_size_t, _P],
    "qs_gather_linear_acc": [_P, _I64, _I64, _P, _INT, _I64, _I64, _P, _P, ctypes.c_size_t, _P],
    "qs_topk_gather_linear_acc": [_P, _I64, _I64, _I64, _P, _INT, _I64, _I64, _P, _P],
    "qs_set_deterministic": [_INT],
    "qs_sparse_linear": [_P, _INT, _I64, _I64, _I64, _P, _INT, _INT, _I64, _P, _INT, _P,
                         ctypes.c_size_t, _P],
    "qs_sparse_linear_pitched": [_P, _INT, _I64, _I64, _I64, _P, _I64, _INT, _INT, _I64, _P,
                                 _INT, _P, ctypes.c_size_t, _P],
    "qs_sparse_linear_backward": [_P, _INT, _I64, _I64, _I64, _P, _INT, _INT, _I64, _P, _INT,
                                  _P, _INT, _P, _INT, _P, ctypes.c_size_t, _P],
    "qs_block_sparse_linear": [_P, _INT, _I64, _I64, _P, _INT, _I64, _P, _INT, _P, _P,
                               ctypes.c_size_t, _P],
    "qs_sparse_moe_ffn": [_P, _INT, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P,
                          _INT, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "qs_sparse_linear_i8t": [_P, _I64, _I64, _I64, _P, ctypes.c_float, _I64, _P, _P, _P, _P,
                             _P, _P, ctypes.c_size_t, _P],
    "qs_sparse_ffn": [_P, _INT, _I64, _I64, _I64, _INT, _I64, _I64, _P, _P, _P, _P, _P, _P,
                      _INT, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "qs_sparse_ffn_pitched": [_P, _INT, _I64, _I64, _I64, _INT, _I64, _I64, _P, _P, _I64, _P,
                              _I64, _P, _P, _P, _INT, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "qs_sparse_ffn_static": [_P, _INT, _I64, _I64, _I64, _INT, _I64, _I64, _P, _P, _P, _P, _P,
                             _P, _INT, _P, _P, _P, _P],
    "qs_workspace_bytes": [_INT, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
    "qs_ternarize": [_P, _I64, _I64, _P, ctypes.POINTER(ctypes.c_float)],
    "qs_pack_ternary": [_P, _I64, _I64, _P],
    "qs_last_error": [],
    "qs_version": [],
}

_lib = None


class QSError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"qs status {status}: {msg}")
        self.status = status


def lib_path() -> str:
    return os.path.join(_HERE, "_lib", "libqs.so")


def load(path: str | None = None):
    """Load libqs.so (built in-tree by sparse_activation_amd.build), or the
    library at `path` in its place (for example the host-sanitized build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m sparse_activation_amd.build`")
    lib = ctypes.CDLL(path)
    for name, argtypes in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_char_p if name in ("qs_last_error", "qs_version") else ctypes.c_int
    _lib = lib
    return lib


def qs_last_error() -> str:
    return load().qs_last_error().decode()


def qs_version() -> str:
    return load().qs_version().decode()


def _check(status: int):
    if status != QS_OK:
        raise QSError(status, qs_last_error())


# ------------------------------------------------------------------ helpers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.int8:
        return I8
    raise TypeError(f"unsupported dtype {t.dtype}")


def _torch_dtype(code: int):
    torch = _torch()
    return {F32: torch.float32, BF16: torch.bfloat16, I8: torch.int8}[code]


def _dev(*ts, strided=()):
    """The common device of the tensors; each must be contiguous, except those
    also listed in `strided` (weights whose row pitch the caller passes on),
    which need contiguous rows."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if any(t is s for s in strided):
            if t.dim() != 2 or t.stride(1) != 1 or t.stride(0) < t.shape[1]:
                raise ValueError("weights must be 2-D with contiguous rows")
        elif not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
    return dev


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _row_pitch(t, name: str) -> int:
    """Elements from one row of the 2-D tensor `t` to the next; its rows must
    be contiguous (a column slice of a wider tensor gives a padded pitch)."""
    if t.dim() != 2 or t.stride(1) != 1 or t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    return int(t.stride(0))


def _stream(dev):
    return ctypes.c_void_p(_torch().cuda.current_stream(dev).cuda_stream)


def qs_workspace_bytes(op: int, rows: int, d: int, n: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load().qs_workspace_bytes(op, rows, d, n, ctypes.byref(out)))
    return int(out.value)


def _workspace(ws, op, rows, d, n, dev):
    need = qs_workspace_bytes(op, rows, d, n)
    if ws is None:
        ws = _torch().empty(max(need, 1), dtype=_torch().uint8, device=dev)
    return ws, ws.numel() * ws.element_size()


# ------------------------------------------------------------------ entry points

def qs_topk_mask(x, k: int, mask=None, idx=None, tau=None, cutoff=None, xs=None,
                 want_mask=True, want_idx=True, want_desc=True, want_xs=False):
    """Per-row top-K by |x| (ties to the lower index).

    Returns (mask, idx, tau, cutoff), plus xs = X (.) M in fp32 when
    want_xs or xs is given."""
    torch = _torch()
    rows, d = x.shape
    dev = _dev(x, mask, idx, tau, cutoff, xs)
    if want_xs and xs is None:
        xs = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if want_mask and mask is None:
        mask = torch.empty((rows, d), dtype=torch.uint8, device=dev)
    if want_idx and idx is None:
        idx = torch.empty((rows, k), dtype=torch.int32, device=dev)
    if want_desc and tau is None:
        tau = torch.empty(rows, dtype=torch.int32, device=dev)      # u32 bits
    if want_desc and cutoff is None:
        cutoff = torch.empty(rows, dtype=torch.int32, device=dev)
    _check(load().qs_topk_mask(_ptr(x), _dtype_code(x), rows, d, k, _ptr(mask), _ptr(idx),
                               _ptr(tau), _ptr(cutoff), _ptr(xs), _stream(dev)))
    if xs is not None:
        return mask, idx, tau, cutoff, xs
    return mask, idx, tau, cutoff


def gather_workspace(rows: int, d_in: int, n_out: int, device=None):
    """A zero-filled workspace for qs_gather_linear (zeroed once, reusable)."""
    torch = _torch()
    need = qs_workspace_bytes(OP_GATHER_LINEAR, rows, d_in, n_out)
    return torch.zeros(max(need, 1), dtype=torch.uint8, device=device or "cuda")


def qs_gather_linear(xs, wt, y=None, y_dtype=None, ws=None):
    """Y = Xs . W^T for a sparsified fp32 Xs; `wt` is W^T [d_in, n_out].

    `ws` must come from gather_workspace() (zeroed once); one is made if None."""
    torch = _torch()
    rows, d_in = xs.shape
    if xs.dtype != torch.float32:
        raise TypeError("xs must be float32")
    if wt.shape[0] != d_in:
        raise ValueError("wt must be [d_in, n_out]")
    n_out = wt.shape[1]
    dev = _dev(xs, wt, y, ws, strided=(wt,))
    if y is None:
        y = torch.empty((rows, n_out), dtype=y_dtype or torch.float32, device=dev)
    if ws is None:
        ws = gather_workspace(rows, d_in, n_out, dev)
    ws_bytes = ws.numel() * ws.element_size()
    _check(load().qs_gather_linear(_ptr(xs), rows, d_in, _ptr(wt), _dtype_code(wt), n_out,
                                   _row_pitch(wt, "wt"), _ptr(y), _dtype_code(y), _ptr(ws),
                                   ws_bytes, _stream(dev)))
    return y


def qs_gather_linear_acc(xs, wt, y, ws=None):
    """Y += Xs . W^T into the fp32 tensor `y` (float atomics across K-splits).

    `ws` as for qs_gather_linear."""
    torch = _torch()
    rows, d_in = xs.shape
    if xs.dtype != torch.float32 or y.dtype != torch.float32:
        raise TypeError("xs and y must be float32")
    if wt.shape[0] != d_in:
        raise ValueError("wt must be [d_in, n_out]")
    n_out = wt.shape[1]
    if tuple(y.shape) != (rows, n_out):
        raise ValueError("y must be [rows, n_out]")
    dev = _dev(xs, wt, y, ws, strided=(wt,))
    if ws is None:
        ws = gather_workspace(rows, d_in, n_out, dev)
    ws_bytes = ws.numel() * ws.element_size()
    _check(load().qs_gather_linear_acc(_ptr(xs), rows, d_in, _ptr(wt), _dtype_code(wt), n_out,
                                       _row_pitch(wt, "wt"), _ptr(y), _ptr(ws), ws_bytes,
                                       _stream(dev)))
    return y


def qs_topk_gather_linear_acc(x, k: int, wt, y):
    """Y += (X (.) M) . W^T into the fp32 tensor `y`, M the per-row top-k mask
    of the fp32 `x` by magnitude, selection and gather in one launch (bf16
    W^T [d_in, n_out]; float atomics across the workgroups)."""
    torch = _torch()
    rows, d_in = x.shape
    if x.dtype != torch.float32 or y.dtype != torch.float32:
        raise TypeError("x and y must be float32")
    if wt.shape[0] != d_in:
        raise ValueError("wt must be [d_in, n_out]")
    n_out = wt.shape[1]
    if tuple(y.shape) != (rows, n_out):
        raise ValueError("y must be [rows, n_out]")
    dev = _dev(x, wt, y, strided=(wt,))
    ldw = _row_pitch(wt, "wt")
    _check(load().qs_topk_gather_linear_acc(_ptr(x), rows, d_in, k, _ptr(wt), _dtype_code(wt),
                                            n_out, ldw, _ptr(y), _stream(dev)))
    return y


def qs_set_deterministic(on: bool) -> bool:
    """Process-wide: fixed-order split-K sums (bitwise reproducible) if on.

    Returns the previous setting."""
    return bool(load().qs_set_deterministic(1 if on else 0))


def qs_sparse_linear(x, k: int, w, layout: int = LAYOUT_WT, y=None, y_dtype=None, ws=None):
    """Y = (X (.) M) . W^T.  `w` is W^T [d_in, n_out] (LAYOUT_WT) or W [n_out, d_in]."""
    torch = _torch()
    rows, d_in = x.shape
    n_out = w.shape[1] if layout == LAYOUT_WT else w.shape[0]
    d_w = w.shape[0] if layout == LAYOUT_WT else w.shape[1]
    if d_w != d_in:
        raise ValueError("weight shape does not match x")
    dev = _dev(x, w, y, ws, strided=(w,) if layout == LAYOUT_WT else ())
    ldw = _row_pitch(w, "w")
    natural = n_out if layout == LAYOUT_WT else d_in
    if y is None:
        y = torch.empty((rows, n_out), dtype=y_dtype or torch.float32, device=dev)
    ws, ws_bytes = _workspace(ws, OP_SPARSE_LINEAR, rows, d_in, n_out, dev)
    if ldw == natural:
        _check(load().qs_sparse_linear(_ptr(x), _dtype_code(x), rows, d_in, k, _ptr(w),
                                       _dtype_code(w), layout, n_out, _ptr(y), _dtype_code(y),
                                       _ptr(ws), ws_bytes, _stream(dev)))
    else:
        _check(load().qs_sparse_linear_pitched(_ptr(x), _dtype_code(x), rows, d_in, k, _ptr(w),
                                               ldw, _dtype_code(w), layout, n_out, _ptr(y),
                                               _dtype_code(y), _ptr(ws), ws_bytes, _stream(dev)))
    return y


def qs_sparse_linear_pitched(x, k: int, w, layout: int = LAYOUT_WT, y=None, y_dtype=None,
                             ws=None):
    """qs_sparse_linear; the row pitch of `w` is taken from its strides (a
    column slice of a wider tensor is a padded W^T)."""
    return qs_sparse_linear(x, k, w, layout, y=y, y_dtype=y_dtype, ws=ws)


def qs_sparse_linear_backward(x, k: int, w, dy, layout: int = LAYOUT_W, want_dx=True,
                              want_dw=True, dx=None, dw=None, out_dtype=None, ws=None):
    """Gradients of Y = (X (.) M) . W^T with the straight-through estimator:
    dX = dY . W (not masked), dW = dY^T . (X (.) M) in the layout of `w`
    (W^T [d_in, n_out] for LAYOUT_WT, W [n_out, d_in] for LAYOUT_W).
    Returns (dx, dw); either is None when not asked for."""
    torch = _torch()
    rows, d_in = x.shape
    n_out = w.shape[1] if layout == LAYOUT_WT else w.shape[0]
    d_w = w.shape[0] if layout == LAYOUT_WT else w.shape[1]
    if d_w != d_in or tuple(dy.shape) != (rows, n_out):
        raise ValueError("shapes of x, w and dy do not match")
    dev = _dev(x, w, dy, dx, dw, ws)
    odt = out_dtype or torch.float32
    if want_dx and dx is None:
        dx = torch.empty((rows, d_in), dtype=odt, device=dev)
    if want_dw and dw is None:
        dw = torch.empty(tuple(w.shape), dtype=odt, device=dev)
    dx = dx if want_dx else None
    dw = dw if want_dw else None
    ws, ws_bytes = _workspace(ws, OP_SPARSE_LINEAR_BACKWARD, rows, d_in, n_out, dev)
    _check(load().qs_sparse_linear_backward(
        _ptr(x), _dtype_code(x), rows, d_in, k, _ptr(w), _dtype_code(w), layout, n_out,
        _ptr(dy), _dtype_code(dy), _ptr(dx), _dtype_code(dx) if dx is not None else F32,
        _ptr(dw), _dtype_code(dw) if dw is not None else F32, _ptr(ws), ws_bytes, _stream(dev)))
    return dx, dw


def qs_block_sparse_linear(x, w, y=None, y_dtype=None, want_mask=False, mask=None, ws=None):
    """Block Q-Sparse linear: Y = (X (.) M) . W^T with M keeping the 2 largest
    |x| of every contiguous block of 4 features (ties to the lower index).
    `w` is W [n_out, d_in].  Returns (y, mask) (mask None unless asked for)."""
    torch = _torch()
    rows, d_in = x.shape
    n_out = w.shape[0]
    if w.shape[1] != d_in:
        raise ValueError("weight shape does not match x")
    dev = _dev(x, w, y, mask, ws)
    if y is None:
        y = torch.empty((rows, n_out), dtype=y_dtype or torch.float32, device=dev)
    if want_mask and mask is None:
        mask = torch.empty((rows, d_in), dtype=torch.uint8, device=dev)
    ws, ws_bytes = _workspace(ws, OP_BLOCK_SPARSE_LINEAR, rows, d_in, n_out, dev)
    _check(load().qs_block_sparse_linear(_ptr(x), _dtype_code(x), rows, d_in, _ptr(w),
                                         _dtype_code(w), n_out, _ptr(y), _dtype_code(y),
                                         _ptr(mask), _ptr(ws), ws_bytes, _stream(dev)))
    return y, mask


def qs_sparse_moe_ffn(x, top_k: int, w_router, w_gate, w_up, w_down_t, b_gate=None, b_up=None,
                      y=None, y_dtype=None, want_all=False, ws=None):
    """Mixture-of-experts dReLU FFN (decode).  Weights are stacked per expert:
    w_router [E, d], w_gate / w_up / w_down_t [E, ffn, d], biases [E, ffn].
    Returns y, or with want_all (y, logits, experts, weights, h)."""
    torch = _torch()
    rows, d = x.shape
    n_exp, ffn = w_gate.shape[0], w_gate.shape[1]
    for t in (w_up, w_down_t):
        if tuple(t.shape) != (n_exp, ffn, d):
            raise ValueError("expert weights must all be [E, ffn, d]")
    if tuple(w_router.shape) != (n_exp, d):
        raise ValueError("w_router must be [E, d]")
    dev = _dev(x, w_router, w_gate, w_up, w_down_t, b_gate, b_up, y, ws)
    if y is None:
        y = torch.empty((rows, d), dtype=y_dtype or torch.float32, device=dev)
    logits = experts = weights = h = None
    if want_all:
        logits = torch.empty((rows, n_exp), dtype=torch.float32, device=dev)
        experts = torch.empty((rows, top_k), dtype=torch.int32, device=dev)
        weights = torch.empty((rows, top_k), dtype=torch.float32, device=dev)
        h = torch.empty((rows, top_k, ffn), dtype=torch.float32, device=dev)
    ws, ws_bytes = _workspace(ws, OP_SPARSE_MOE_FFN, rows * top_k, d, ffn, dev)
    _check(load().qs_sparse_moe_ffn(
        _ptr(x), _dtype_code(x), rows, d, ffn, n_exp, top_k, _ptr(w_router), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down_t), _ptr(b_gate), _ptr(b_up), _ptr(y), _dtype_code(y),
        _ptr(logits), _ptr(experts), _ptr(weights), _ptr(h), _ptr(ws), ws_bytes, _stream(dev)))
    if want_all:
        return y, logits, experts, weights, h
    return y


def qs_sparse_linear_i8t(x, k: int, wt_packed, alpha: float, n_out: int, acc=None, y=None,
                         xq=None, xscale=None, idx=None, ws=None, want_all=True):
    """Quantised Q-Sparse linear; returns (acc, y, xq, xscale, idx)."""
    torch = _torch()
    rows, d_in = x.shape
    if tuple(wt_packed.shape) != (d_in, n_out // 4):
        raise ValueError("wt_packed must be [d_in, n_out/4]")
    dev = _dev(x, wt_packed, acc, y, xq, xscale, idx, ws)
    if want_all:
        acc = acc if acc is not None else torch.empty((rows, n_out), dtype=torch.int32, device=dev)
        y = y if y is not None else torch.empty((rows, n_out), dtype=torch.float32, device=dev)
        xq = xq if xq is not None else torch.empty((rows, d_in), dtype=torch.int8, device=dev)
        xscale = xscale if xscale is not None else torch.empty(rows, dtype=torch.float32, device=dev)
        idx = idx if idx is not None else torch.empty((rows, k), dtype=torch.int32, device=dev)
    ws, ws_bytes = _workspace(ws, OP_SPARSE_LINEAR_I8T, rows, d_in, n_out, dev)
    _check(load().qs_sparse_linear_i8t(_ptr(x), rows, d_in, k, _ptr(wt_packed),
                                       ctypes.c_float(alpha), n_out, _ptr(acc), _ptr(y),
                                       _ptr(xq), _ptr(xscale), _ptr(idx), _ptr(ws), ws_bytes,
                                       _stream(dev)))
    return acc, y, xq, xscale, idx


def qs_sparse_ffn(x, act: int, k_in: int, k_mid: int, w_up, w_down_t, w_gate=None,
                  b_gate=None, b_up=None, y=None, y_dtype=None, h=None, mid_idx=None,
                  mid_cnt=None, ws=None, want_h=False, want_mid=False):
    """Sparse FFN (squared ReLU, dReLU or gated squared ReLU); returns (y, h, mid_idx, mid_cnt)."""
    torch = _torch()
    rows, d = x.shape
    ffn = w_down_t.shape[0]
    dev = _dev(x, w_up, w_down_t, w_gate, b_gate, b_up, y, h, mid_idx, mid_cnt, ws,
               strided=(w_up, w_down_t, w_gate))
    if y is None:
        y = torch.empty((rows, d), dtype=y_dtype or torch.float32, device=dev)
    if want_h and h is None:
        h = torch.empty((rows, ffn), dtype=torch.float32, device=dev)
    if want_mid and mid_idx is None:
        mid_idx = torch.empty((rows, ffn), dtype=torch.int32, device=dev)
    if want_mid and mid_cnt is None:
        mid_cnt = torch.empty(rows, dtype=torch.int32, device=dev)
    op = {ACT_RELU2: OP_SPARSE_FFN_RELU2, ACT_DRELU: OP_SPARSE_FFN_DRELU,
          ACT_RELU2_GLU: OP_SPARSE_FFN_RELU2_GLU}.get(act, OP_SPARSE_FFN_RELU2)
    ws, ws_bytes = _workspace(ws, op, rows, d, ffn, dev)
    ld_up, ld_down = _row_pitch(w_up, "w_up"), _row_pitch(w_down_t, "w_down_t")
    if w_gate is not None and _row_pitch(w_gate, "w_gate") != ld_up:
        raise ValueError("w_gate and w_up must have the same row pitch")
    if (ld_up, ld_down) == (d if act == ACT_DRELU else ffn, d):
        _check(load().qs_sparse_ffn(_ptr(x), _dtype_code(x), rows, d, ffn, act, k_in, k_mid,
                                    _ptr(w_gate), _ptr(w_up), _ptr(w_down_t), _ptr(b_gate),
                                    _ptr(b_up), _ptr(y), _dtype_code(y), _ptr(h), _ptr(mid_idx),
                                    _ptr(mid_cnt), _ptr(ws), ws_bytes, _stream(dev)))
    else:
        _check(load().qs_sparse_ffn_pitched(
            _ptr(x), _dtype_code(x), rows, d, ffn, act, k_in, k_mid, _ptr(w_gate), _ptr(w_up),
            ld_up, _ptr(w_down_t), ld_down, _ptr(b_gate), _ptr(b_up), _ptr(y), _dtype_code(y),
            _ptr(h), _ptr(mid_idx), _ptr(mid_cnt), _ptr(ws), ws_bytes, _stream(dev)))
    return y, h, mid_idx, mid_cnt


def qs_sparse_ffn_pitched(x, act: int, k_in: int, k_mid: int, w_up, w_down_t, **kw):
    """qs_sparse_ffn; the row pitches of the weights are taken from their
    strides (column slices of wider tensors are padded rows)."""
    return qs_sparse_ffn(x, act, k_in, k_mid, w_up, w_down_t, **kw)


def qs_sparse_ffn_static(x, act: int, k_in: int, k_mid: int, w_up, w_down_t, w_gate=None,
                         b_gate=None, b_up=None, y=None, y_dtype=None, h=None, mid_idx=None,
                         mid_cnt=None, want_h=False, want_mid=False):
    """qs_sparse_ffn on the library's per-GPU scratch array (no workspace is
    allocated); returns (y, h, mid_idx, mid_cnt)."""
    torch = _torch()
    rows, d = x.shape
    ffn = w_down_t.shape[0]
    dev = _dev(x, w_up, w_down_t, w_gate, b_gate, b_up, y, h, mid_idx, mid_cnt)
    if y is None:
        y = torch.empty((rows, d), dtype=y_dtype or torch.float32, device=dev)
    if want_h and h is None:
        h = torch.empty((rows, ffn), dtype=torch.float32, device=dev)
    if want_mid and mid_idx is None:
        mid_idx = torch.empty((rows, ffn), dtype=torch.int32, device=dev)
    if want_mid and mid_cnt is None:
        mid_cnt = torch.empty(rows, dtype=torch.int32, device=dev)
    up_len = d if act == ACT_DRELU else ffn
    if (_row_pitch(w_up, "w_up"), _row_pitch(w_down_t, "w_down_t")) != (up_len, d) or (
            w_gate is not None and _row_pitch(w_gate, "w_gate") != up_len):
        raise ValueError("qs_sparse_ffn_static takes unpadded weights")
    _check(load().qs_sparse_ffn_static(_ptr(x), _dtype_code(x), rows, d, ffn, act, k_in, k_mid,
                                       _ptr(w_gate), _ptr(w_up), _ptr(w_down_t), _ptr(b_gate),
                                       _ptr(b_up), _ptr(y), _dtype_code(y), _ptr(h),
                                       _ptr(mid_idx), _ptr(mid_cnt), _stream(dev)))
    return y, h, mid_idx, mid_cnt


def qs_ternarize(w_host):
    """Host-side ternary quantisation: returns (t int8 numpy [n_out, d_in], alpha float)."""
    import numpy as np
    w = np.ascontiguousarray(w_host, dtype=np.float32)
    n_out, d_in = w.shape
    t = np.empty_like(w, dtype=np.int8)
    alpha = ctypes.c_float(0.0)
    _check(load().qs_ternarize(w.ctypes.data_as(ctypes.c_void_p), n_out, d_in,
                               t.ctypes.data_as(ctypes.c_void_p), ctypes.byref(alpha)))
    return t, float(alpha.value)


def qs_pack_ternary(t_host):
    """Host-side packing of t [n_out, d_in] into the 2-bit W^T layout [d_in, n_out/4]."""
    import numpy as np
    t = np.ascontiguousarray(t_host, dtype=np.int8)
    n_out, d_in = t.shape
    packed = np.empty((d_in, n_out // 4), dtype=np.uint8)
    _check(load().qs_pack_ternary(t.ctypes.data_as(ctypes.c_void_p), n_out, d_in,
                                  packed.ctypes.data_as(ctypes.c_void_p)))
    return packed
