"""Plain, slow CPU definitions of the Q-Sparse inference forward.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Conventions
-----------
* ``X`` is ``[R, D]``: R tokens (rows), D input features.
* ``W`` is given in the nn.Linear layout ``[N, D]`` and the product is
  ``Y = X . W^T`` (Q-Sparse news article, "Sparsification with the Top-K
  function": every attention and FFN projection is such a product).
* Floating-point results are float64 sums of exact products of the inputs
  (bf16 and fp32 inputs convert to float64 exactly).
"""
from __future__ import annotations

import math

import numpy as np

EPS = np.float32(1e-5)


# ---------------------------------------------------------------------------
# Top-K selection
# ---------------------------------------------------------------------------

def magnitude(x) -> np.ndarray:
    """|x| as float64, exact for fp32/bf16/int inputs.  +0 and -0 both give 0."""
    return np.abs(np.asarray(x, dtype=np.float64))


def topk_select(mag, k: int):
    """Per-row top-K by magnitude, ties going to the lower index.

    Q-Sparse news article, "Sparsification with the Top-K function": take |X|,
    sort it, keep the K entries of largest magnitude, and build a binary mask
    of the same shape as X that is 1 at those positions and 0 elsewhere; K is
    a preset hyperparameter.  The pages say nothing about ties; the reading
    taken is that among equal magnitudes the lower feature index wins, which
    makes the selected set unique.  Selection is per token (row).

    Step by step: sort each row by (magnitude descending, index ascending)
    with NumPy's lexsort, take the first K positions.

    Returns ``(mask u8 [R,D], idx i32 [R,K] ascending, tau f64 [R],
    cutoff i32 [R])`` where tau is the magnitude of the K-th selected entry
    and ``cutoff`` is one past the index of the last selected entry whose
    magnitude equals tau, so that entry j is selected iff
    ``mag[j] > tau or (mag[j] == tau and j < cutoff)``.  For K = 0, tau is
    +inf and cutoff is 0.
    """
    mag = np.asarray(mag, dtype=np.float64)
    if mag.ndim != 2:
        raise ValueError("mag must be [R, D]")
    rows, d = mag.shape
    if not 0 <= k <= d:
        raise ValueError("need 0 <= k <= D")
    mask = np.zeros((rows, d), dtype=np.uint8)
    idx = np.zeros((rows, k), dtype=np.int32)
    tau = np.full(rows, np.inf)
    cutoff = np.zeros(rows, dtype=np.int32)
    j = np.arange(d)
    for r in range(rows):
        order = np.lexsort((j, -mag[r]))   # primary: -mag ascending; then j
        sel = order[:k]
        mask[r, sel] = 1
        idx[r] = np.sort(sel)
        if k > 0:
            tau[r] = mag[r, order[k - 1]]
            ties = sel[mag[r, sel] == tau[r]]
            cutoff[r] = int(ties.max()) + 1
    return mask, idx, tau, cutoff


def block_topk_select(mag, n_keep: int, block: int):
    """Block Q-Sparse selection: top-``n_keep`` by magnitude inside every
    contiguous block of ``block`` features of each row, ties to the lower
    index (an N:M pattern, N = n_keep, M = block).

    Q-Sparse abstract (the arXiv 2407.10969 listing page, authors' English
    abstract) introduces Block Q-Sparse for batch training and inference; the
    same page's machine-written Chinese summary (method details, key-design
    item 3) says only that the activations are divided into blocks to use the
    hardware better.  Neither gives the rule, so this is a reading:
    the top-K of the Top-K section applied within each block of contiguous
    features of a token, with K = n_keep per block, which is the N:M
    structured pattern that sparse matrix cores accept (2:4 on the MI355X).

    Step by step: for each block, sort its magnitudes by (magnitude
    descending, index ascending) and keep the first n_keep.  Returns the u8
    mask [R, D].  D must be a multiple of ``block``.
    """
    mag = np.asarray(mag, dtype=np.float64)
    rows, d = mag.shape
    if d % block != 0 or not 0 <= n_keep <= block:
        raise ValueError("D must be a multiple of block and 0 <= n_keep <= block")
    mask = np.zeros((rows, d), dtype=np.uint8)
    j = np.arange(block)
    for r in range(rows):
        for b0 in range(0, d, block):
            order = np.lexsort((j, -mag[r, b0:b0 + block]))
            mask[r, b0 + order[:n_keep]] = 1
    return mask


# ---------------------------------------------------------------------------
# Sparse-activation linear
# ---------------------------------------------------------------------------

def sparse_linear(x, w, mask):
    """Y = (X (.) M) . W^T in float64, and the error scale T = |X (.) M| . |W|^T.

    Q-Sparse news article, "Sparsification with the Top-K function": the
    Hadamard product of X with the mask replaces X in the following product;
    since most of its entries are zero the product needs far less compute and
    memory traffic (Q-Sparse aibase report: I/O is the main inference
    bottleneck).  A library matmul is used as the product step.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    m = np.asarray(mask).astype(bool)
    xs = np.where(m, x, 0.0)
    y = xs @ w.T
    t = np.abs(xs) @ np.abs(w).T
    return y, t


# ---------------------------------------------------------------------------
# FFN activations
# ---------------------------------------------------------------------------

def relu2(u):
    """Squared ReLU: relu(u)^2 (Q-Sparse news article, end of the Top-K
    section: the FFN uses squared ReLU to raise activation sparsity).  The
    un-gated form is the reading taken; the formula itself is missing."""
    u = np.asarray(u, dtype=np.float64)
    r = np.maximum(u, 0.0)
    return r * r


def relu2_glu(g, u):
    """Gated squared ReLU: relu(gate)^2 (.) up (Q-Sparse news article, end of
    the Top-K section: squared ReLU in the FFN, with (.) the Hadamard
    product).  The gated reading of that sentence; h keeps the sign of up."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    r = np.maximum(g, 0.0)
    return (r * r) * u


def drelu(g, u):
    """dReLU: relu(gate) (.) relu(up) (Turbo Sparse summary, Eq. 2: ReLU is
    applied after both the gate and the up projection)."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    return np.maximum(g, 0.0) * np.maximum(u, 0.0)


def ffn_relu2(x, k_in, w_up, k_mid, w_down):
    """Squared-ReLU FFN with top-K on the input and top-K on the intermediate.

    Steps: mask1 = top-K(|x|, k_in); u = (x (.) mask1) . W_up^T;
    h = relu(u)^2; mask2 = top-K(|h|, k_mid) (Turbo Sparse summary, Eq. 3-4:
    top-k% of the activation by absolute value before W_down);
    y = (h (.) mask2) . W_down^T.  Returns every stage.
    """
    m1, idx1, tau1, cut1 = topk_select(magnitude(x), k_in)
    u, t_u = sparse_linear(x, w_up, m1)
    h = relu2(u)
    m2, idx2, tau2, cut2 = topk_select(magnitude(h), k_mid)
    y, t_y = sparse_linear(h, w_down, m2)
    return dict(mask1=m1, idx1=idx1, tau1=tau1, cutoff1=cut1, u=u, T_u=t_u,
                h=h, mask2=m2, idx2=idx2, tau2=tau2, cutoff2=cut2, y=y, T_y=t_y)


def ffn_relu2_down_from(h, k_mid, w_down):
    """Second half of ``ffn_relu2`` started from a given intermediate h
    (used to check a device's down projection against its own h)."""
    m2, idx2, tau2, cut2 = topk_select(magnitude(h), k_mid)
    y, t_y = sparse_linear(h, w_down, m2)
    return dict(mask2=m2, idx2=idx2, tau2=tau2, cutoff2=cut2, y=y, T_y=t_y)


def ffn_relu2_glu(x, k_in, w_gate, w_up, k_mid, w_down):
    """Gated squared-ReLU FFN with top-K on the input and on the intermediate.

    Steps: mask1 = top-K(|x|, k_in) (the same sparse input feeds both
    projections); g = (x (.) mask1) . W_gate^T; u = (x (.) mask1) . W_up^T;
    h = relu(g)^2 (.) u; mask2 = top-K(|h|, k_mid); y = (h (.) mask2) .
    W_down^T (Turbo Sparse summary, Eq. 3-4, for the top-k% by magnitude
    before W_down).  Returns every stage.
    """
    m1, idx1, tau1, cut1 = topk_select(magnitude(x), k_in)
    g, t_g = sparse_linear(x, w_gate, m1)
    u, t_u = sparse_linear(x, w_up, m1)
    h = relu2_glu(g, u)
    m2, idx2, tau2, cut2 = topk_select(magnitude(h), k_mid)
    y, t_y = sparse_linear(h, w_down, m2)
    return dict(mask1=m1, idx1=idx1, tau1=tau1, cutoff1=cut1, g=g, T_g=t_g, u=u, T_u=t_u,
                h=h, mask2=m2, idx2=idx2, tau2=tau2, cutoff2=cut2, y=y, T_y=t_y)


def ffn_drelu(x, w_gate, b_gate, w_up, b_up, w_down):
    """dReLU FFN whose down projection gathers only the nonzero neurons.

    g = x . W_gate^T + b_gate; u = x . W_up^T + b_up (biases added after the
    full sums); h = relu(g) (.) relu(u) (Turbo Sparse summary, Eq. 2);
    N = {i : h_i != 0} ascending; y = sum over i in N of h_i . W_down[:, i].
    The input is not top-K'd.  Returns every stage, with the error scales
    T_g, T_u (including |b|) and T_y.
    """
    x = np.asarray(x, dtype=np.float64)
    wg = np.asarray(w_gate, dtype=np.float64)
    wu = np.asarray(w_up, dtype=np.float64)
    bg = np.zeros(wg.shape[0]) if b_gate is None else np.asarray(b_gate, np.float64)
    bu = np.zeros(wu.shape[0]) if b_up is None else np.asarray(b_up, np.float64)
    g = x @ wg.T + bg
    u = x @ wu.T + bu
    t_g = np.abs(x) @ np.abs(wg).T + np.abs(bg)
    t_u = np.abs(x) @ np.abs(wu).T + np.abs(bu)
    h = drelu(g, u)
    out = ffn_drelu_down_from(h, w_down)
    out.update(g=g, u=u, T_g=t_g, T_u=t_u, h=h)
    return out


def moe_route(x, w_router, top_k: int):
    """Top-k expert routing of every token.

    Turbo Sparse summary (per-layer zero-activation passage): the MoE model
    activates 2 of its 8 experts per layer, and each expert FFN keeps only
    ~15% of its neurons active after dReLU.  The routing rule is not on the
    pages; the reading taken is the usual one for that model family:
    logits = x . W_router^T, keep the top_k logits of each token (ties to the
    lower expert index, the same rule as the activation top-K), and weight
    the chosen experts by a softmax over the kept logits only.

    Returns (logits f64 [R, E], experts i32 [R, top_k] ascending,
    weights f64 [R, top_k] matching experts, T_logits scale).
    """
    x = np.asarray(x, dtype=np.float64)
    wr = np.asarray(w_router, dtype=np.float64)
    logits = x @ wr.T
    t_logits = np.abs(x) @ np.abs(wr).T
    rows, e = logits.shape
    if not 1 <= top_k <= e:
        raise ValueError("need 1 <= top_k <= n_experts")
    experts = np.zeros((rows, top_k), dtype=np.int32)
    weights = np.zeros((rows, top_k))
    for r in range(rows):
        order = np.lexsort((np.arange(e), -logits[r]))
        sel = np.sort(order[:top_k])
        z = logits[r, sel] - logits[r, sel].max()
        p = np.exp(z)
        experts[r] = sel
        weights[r] = p / p.sum()
    return logits, experts, weights, t_logits


def moe_drelu_ffn(x, w_router, top_k, w_gate, b_gate, w_up, b_up, w_down, experts=None,
                  weights=None):
    """Mixture-of-experts dReLU FFN: y = sum over the token's chosen experts e
    of weight_e * FFN_e(x), FFN_e the dReLU FFN of expert e (ffn_drelu, whose
    down projection gathers only the nonzero neurons).

    Turbo Sparse summary: 2 of 8 experts per layer and ~85% of each expert's
    neurons inactive, so ~3% of the layer's parameters are used per token.
    Expert weights are stacked: w_gate, w_up [E, ffn, d], w_down [E, d, ffn]
    (nn.Linear layout of the down projection, as ffn_drelu takes it), biases
    [E, ffn] or None.  `experts`/`weights` override the routing (stage-wise
    checks feed the routing a device produced).  Returns the routing, every
    pair's hidden h [R, top_k, ffn] and down output, y and its scale T_y
    (sum of weight * T_y over the pairs).
    """
    x = np.asarray(x, dtype=np.float64)
    logits, ex, wts, t_logits = moe_route(x, w_router, top_k)
    if experts is not None:
        ex = np.asarray(experts, dtype=np.int32)
        wts = np.asarray(weights, dtype=np.float64)
    rows = x.shape[0]
    d = x.shape[1]
    ffn = np.asarray(w_gate[0]).shape[0]
    h = np.zeros((rows, top_k, ffn))
    g = np.zeros((rows, top_k, ffn))
    u = np.zeros((rows, top_k, ffn))
    t_g = np.zeros((rows, top_k, ffn))
    t_u = np.zeros((rows, top_k, ffn))
    y_pair = np.zeros((rows, top_k, d))
    t_pair = np.zeros((rows, top_k, d))
    for r in range(rows):
        for j in range(top_k):
            e = int(ex[r, j])
            out = ffn_drelu(x[r:r + 1], w_gate[e], None if b_gate is None else b_gate[e],
                            w_up[e], None if b_up is None else b_up[e], w_down[e])
            h[r, j], g[r, j], u[r, j] = out["h"][0], out["g"][0], out["u"][0]
            t_g[r, j], t_u[r, j] = out["T_g"][0], out["T_u"][0]
            y_pair[r, j], t_pair[r, j] = out["y"][0], out["T_y"][0]
    y = np.einsum("rj,rjd->rd", wts, y_pair)
    t_y = np.einsum("rj,rjd->rd", np.abs(wts), t_pair)
    return dict(logits=logits, T_logits=t_logits, experts=ex, weights=wts, g=g, u=u,
                T_g=t_g, T_u=t_u, h=h, y_pair=y_pair, T_pair=t_pair, y=y, T_y=t_y)


def ffn_drelu_down_from(h, w_down):
    """Nonzero lists of h and the gathered down projection."""
    h = np.asarray(h, dtype=np.float64)
    nz = h != 0.0
    counts = nz.sum(axis=1).astype(np.int32)
    lists = [np.nonzero(nz[r])[0].astype(np.int32) for r in range(h.shape[0])]
    y, t_y = sparse_linear(h, w_down, nz)
    return dict(nz_mask=nz.astype(np.uint8), nz_count=counts, nz_idx=lists, y=y, T_y=t_y)


# ---------------------------------------------------------------------------
# Quantised variant
# ---------------------------------------------------------------------------

def absmax_quant_i8(x):
    """Per-token 8-bit absmax quantisation of the activations, applied before
    top-K (Q-Sparse news article, Top-K section: inputs are quantised first,
    with a small epsilon guarding the denominator).

    The formula is missing from the pages (parity to it is unpinned); the
    reading taken is symmetric absmax to 127 in IEEE binary32 with
    round-to-nearest-even at every step:
    gamma = max |x|; s = 127 / (gamma + eps); q = clamp(rint(x * s), -128, 127).
    Returns ``(q int8 [R,D], s float32 [R], gamma float32 [R])``.
    """
    x = np.asarray(x, dtype=np.float32)
    gamma = np.max(np.abs(x), axis=1)                       # exact
    s = (np.float32(127.0) / (gamma + EPS)).astype(np.float32)
    prod = (x * s[:, None]).astype(np.float32)              # binary32 RN
    q = np.clip(np.rint(prod), -128, 127).astype(np.int8)   # half to even
    return q, s, gamma


def ternarize(w):
    """Ternary weight quantisation with alpha = mean |W| over the whole tensor
    (Q-Sparse news article, Top-K section, the quantiser for 1-bit weights;
    the model is BitNet b1.58, so the values are {-1, 0, +1}).

    The formula is missing from the pages (parity to it is unpinned); the
    reading taken: alpha = fl32(fsum(|w|) / n) (exact sum, float64 divide,
    rounded once more to binary32), t = clamp(rint(w / (alpha + eps)), -1, 1)
    in binary32.  The effective weight is alpha * t.
    """
    w = np.asarray(w, dtype=np.float32)
    total = math.fsum(np.abs(w).astype(np.float64).ravel().tolist())
    alpha = np.float32(total / w.size)
    ratio = (w / (alpha + EPS)).astype(np.float32)
    t = np.clip(np.rint(ratio), -1, 1).astype(np.int8)
    return t, alpha


def unpack_ternary(packed, n_out: int):
    """Decode the packed transposed ternary layout back to t [n_out, d_in].

    Layout: u8 [d_in, n_out/4]; byte c/4 of feature row j holds columns
    c..c+3, column c+i in bits 2i..2i+1, as a 2-bit two's-complement value
    (00 = 0, 01 = +1, 11 = -1; 10 never occurs).
    """
    packed = np.asarray(packed, dtype=np.uint8)
    d_in = packed.shape[0]
    t = np.zeros((n_out, d_in), dtype=np.int8)
    for i in range(4):
        code = (packed >> (2 * i)) & 3                      # [d_in, n_out/4]
        val = np.where(code == 1, 1, np.where(code == 3, -1, 0)).astype(np.int8)
        if np.any(code == 2):
            raise ValueError("invalid ternary code 10")
        t[i::4, :] = val.T
    return t


def i8t_linear(q, s, t, alpha, mask):
    """Quantised Q-Sparse linear: int8 activations x ternary weights.

    acc[r,o] = sum over selected j of q[r,j] * t[o,j], computed exactly in
    integers; y[r,o] = fl32(fl32(acc) * fl32(alpha / s[r])), so that
    y ~= (q / s) . (alpha t)^T.  Returns ``(acc int64, y float32)``.
    """
    q = np.asarray(q, dtype=np.int64)
    t = np.asarray(t, dtype=np.int64)
    m = np.asarray(mask).astype(bool)
    qs = np.where(m, q, 0)
    acc = qs @ t.T                                           # exact integers
    scale = (np.float32(alpha) / np.asarray(s, np.float32)).astype(np.float32)
    y = (acc.astype(np.float32) * scale[:, None]).astype(np.float32)
    return acc, y


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

def ste_backward(grad_y):
    """Straight-through estimator for top-K: the gradient w.r.t. the
    sparsified tensor is copied unchanged to the dense input, including at
    masked positions (Q-Sparse news article, Top-K section, STE passage)."""
    return np.array(grad_y, copy=True)


def sparse_linear_backward(x, w, mask, grad_y):
    """Gradients of Y = (X (.) M) . W^T, given dL/dY, with the top-K
    treated by the straight-through estimator.

    Q-Sparse news article, "Sparsification with the Top-K function", the
    back-propagation passage: the top-K has a zero gradient almost everywhere,
    so Q-Sparse computes the gradient with respect to the sparsified tensor
    and copies it unchanged to the tensor before sparsification.  Through the
    linear map (plain chain rule):

        dXs = dY . W           gradient w.r.t. X (.) M   ([R, N] . [N, D])
        dX  = dXs              the STE copy: no mask, masked-out entries keep
                               their gradient (ste_backward)
        dW  = dY^T . (X (.) M) ([N, R] . [R, D]); column j is zero unless some
                               row selected feature j

    Returns float64 dx [R, D], dw [N, D] and the error scales
    T_dx = |dY| . |W| and T_dw = |dY|^T . |X (.) M| (sums of the absolute
    products, for tolerances).  Library matmuls serve as the product steps.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    gy = np.asarray(grad_y, dtype=np.float64)
    m = np.asarray(mask).astype(bool)
    xs = np.where(m, x, 0.0)
    dxs = gy @ w
    dx = ste_backward(dxs)
    dw = gy.T @ xs
    t_dx = np.abs(gy) @ np.abs(w)
    t_dw = np.abs(gy).T @ np.abs(xs)
    return dict(dx=dx, T_dx=t_dx, dw=dw, T_dw=t_dw)
