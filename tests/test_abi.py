"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its argument validation, workspace sizing and host-side weight preparation
behave as include/qs.h states.  No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import sparse_activation_amd as qs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "qs.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qs_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = qs.load()
    names = _declared()
    assert "qs_sparse_ffn" in names and len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert "gfx950" in qs.qs_version()


FAKE = ctypes.c_void_p(0x1000)          # never dereferenced: every call below fails validation
MISALIGNED = ctypes.c_void_p(0x1004)


def _status(call):
    return call


def test_topk_validation():
    lib = qs.load()
    assert lib.qs_topk_mask(FAKE, qs.F32, 2, 8, 9, None, None, None, None, None, None) == 1
    assert lib.qs_topk_mask(FAKE, qs.F32, 2, 8, -1, None, None, None, None, None, None) == 1
    assert lib.qs_topk_mask(FAKE, 7, 2, 8, 3, None, None, None, None, None, None) == 2
    assert lib.qs_topk_mask(None, qs.F32, 2, 8, 3, None, None, None, None, None, None) == 1
    assert lib.qs_topk_mask(MISALIGNED, qs.F32, 2, 8, 3, None, None, None, None, None,
                            None) == 2
    assert "aligned" in qs.qs_last_error()
    assert lib.qs_topk_mask(FAKE, qs.I8, 2, 8, 3, None, None, None, None, FAKE, None) == 2
    # rows == 0 is a no-op that touches nothing
    assert lib.qs_topk_mask(None, qs.F32, 0, 8, 3, None, None, None, None, None, None) == 0
    assert qs.qs_last_error() == ""


def test_linear_validation_and_workspace():
    lib = qs.load()
    need = qs.qs_workspace_bytes(qs.OP_SPARSE_LINEAR, 4, 1024, 512)
    assert need > 0
    args = lambda **kw: dict(dict(x=FAKE, xt=qs.BF16, rows=4, d=1024, k=100, w=FAKE,
                                  wt=qs.BF16, lay=qs.LAYOUT_WT, n=512, y=FAKE, yt=qs.F32,
                                  ws=FAKE, wsb=need), **kw)

    def call(a):
        return lib.qs_sparse_linear(a["x"], a["xt"], a["rows"], a["d"], a["k"], a["w"],
                                    a["wt"], a["lay"], a["n"], a["y"], a["yt"], a["ws"],
                                    a["wsb"], None)
    assert call(args(k=1025)) == 1
    assert call(args(n=500)) == 2                      # n_out % 8 for bf16 weights
    assert call(args(wsb=need - 1)) == 3
    assert call(args(ws=None)) == 3
    assert call(args(y=None)) == 1
    assert call(args(w=MISALIGNED)) == 2
    assert call(args(lay=qs.LAYOUT_W, xt=qs.F32, wt=qs.F32, n=512)) == 2
    assert call(args(xt=qs.I8)) == 2
    assert call(args(rows=0, x=None, w=None, y=None, ws=None)) == 0


def test_gather_linear_validation():
    lib = qs.load()
    need = qs.qs_workspace_bytes(qs.OP_GATHER_LINEAR, 2, 512, 256)
    assert need >= 16384
    assert lib.qs_gather_linear(FAKE, 2, 512, FAKE, qs.BF16, 252, 252, FAKE, qs.F32, FAKE, need,
                                None) == 2
    assert lib.qs_gather_linear(FAKE, 2, 512, FAKE, qs.BF16, 256, 256, FAKE, qs.F32, FAKE, need - 1,
                                None) == 3
    assert lib.qs_gather_linear(None, 2, 512, FAKE, qs.BF16, 256, 256, FAKE, qs.F32, FAKE, need,
                                None) == 1
    assert lib.qs_gather_linear(FAKE, 2, 512, FAKE, qs.BF16, 256, 252, FAKE, qs.F32, FAKE, need,
                                None) == 1   # ldw < n_out
    assert lib.qs_gather_linear(FAKE, 2, 512, FAKE, qs.BF16, 256, 260, FAKE, qs.F32, FAKE, need,
                                None) == 1   # ldw % 8


def test_gather_linear_acc_validation():
    """Y += Xs . W^T takes qs_gather_linear's workspace and checks; fp32 weights
    in 16-token tiles have no accumulate form."""
    lib = qs.load()
    need = qs.qs_workspace_bytes(qs.OP_GATHER_LINEAR, 2, 512, 256)
    assert lib.qs_gather_linear_acc(FAKE, 2, 512, FAKE, qs.BF16, 252, 252, FAKE, FAKE, need, None) == 2
    assert lib.qs_gather_linear_acc(FAKE, 2, 512, FAKE, qs.BF16, 256, 256, FAKE, FAKE, need - 1,
                                    None) == 3
    assert lib.qs_gather_linear_acc(None, 2, 512, FAKE, qs.BF16, 256, 256, FAKE, FAKE, need, None) == 1
    need16 = qs.qs_workspace_bytes(qs.OP_GATHER_LINEAR, 16, 512, 256)
    assert lib.qs_gather_linear_acc(FAKE, 16, 512, FAKE, qs.F32, 256, 256, FAKE, FAKE, need16,
                                    None) == 2
    assert "8 rows" in qs.qs_last_error()


def test_topk_gather_linear_acc_validation():
    """Selection-in-gather accumulate: bf16 W^T only, d_in % 4 == 0 and <= 16384,
    n_out % 8 == 0, 0 <= k <= d_in, a row pitch ldw >= n_out that is a multiple
    of 8, no workspace; rows == 0 is a no-op."""
    lib = qs.load()
    f = lib.qs_topk_gather_linear_acc
    assert f(FAKE, 1, 11008, 4403, FAKE, qs.F32, 4096, 4096, FAKE, None) == 2     # fp32 W^T
    assert f(FAKE, 1, 11006, 4403, FAKE, qs.BF16, 4096, 4096, FAKE, None) == 2    # d_in % 4
    assert f(FAKE, 1, 16388, 4403, FAKE, qs.BF16, 4096, 4096, FAKE, None) == 2    # d_in too large
    assert f(FAKE, 1, 11008, 4403, FAKE, qs.BF16, 4092, 4092, FAKE, None) == 2    # n_out % 8
    assert f(FAKE, 1, 11008, 11009, FAKE, qs.BF16, 4096, 4096, FAKE, None) == 1   # k > d_in
    assert f(FAKE, 1, 11008, -1, FAKE, qs.BF16, 4096, 4096, FAKE, None) == 1
    assert f(None, 1, 11008, 4403, FAKE, qs.BF16, 4096, 4096, FAKE, None) == 1
    assert f(MISALIGNED, 1, 11008, 4403, FAKE, qs.BF16, 4096, 4096, FAKE, None) == 2
    assert f(FAKE, 65536, 11008, 4403, FAKE, qs.BF16, 4096, 4096, FAKE, None) == 2
    assert f(FAKE, 1, 11008, 4403, FAKE, qs.BF16, 4096, 4092, FAKE, None) == 1  # ldw < n_out
    assert f(FAKE, 1, 11008, 4403, FAKE, qs.BF16, 4096, 4100, FAKE, None) == 1  # ldw % 8
    assert f(FAKE, 1, 11008, 4403, FAKE, qs.BF16, 4096, 1 << 17, FAKE, None) == 2  # > 1 GiB
    assert f(None, 0, 11008, 4403, None, qs.BF16, 4096, 4096, None, None) == 0


def test_pitched_entry_points_validation():
    """Row pitches: at least the row length, a multiple of 8, the padded matrix
    under 1 GiB; dReLU's W_gate / W_up and the dense layout take natural rows
    only.  Every call below fails validation (nothing is enqueued)."""
    lib = qs.load()
    big = ctypes.c_size_t(1 << 40)
    ffn_p = lib.qs_sparse_ffn_pitched

    def ffn(act, ld_up, ld_down, gate=None):
        return ffn_p(FAKE, qs.BF16, 2, 4096, 11008, act, 1638, 4403, gate, FAKE, ld_up, FAKE,
                     ld_down, None, None, FAKE, qs.F32, None, None, None, FAKE, big, None)
    assert ffn(qs.ACT_RELU2, 11000, 4160) == 1                # ld_up < ffn
    assert ffn(qs.ACT_RELU2, 11072, 4100) == 1                # ld_down % 8
    assert ffn(qs.ACT_RELU2, 11072, 4088) == 1                # ld_down < d
    assert ffn(qs.ACT_DRELU, 4160, 4160, gate=FAKE) == 2      # dReLU W_up padded
    assert "natural rows" in qs.qs_last_error()
    assert ffn(qs.ACT_RELU2, 1 << 17, 4160) == 2              # padded W_up^T >= 1 GiB
    assert "1 GiB" in qs.qs_last_error()
    lin = lib.qs_sparse_linear_pitched

    def linear(ldw, layout=qs.LAYOUT_WT):
        return lin(FAKE, qs.BF16, 2, 4096, 1638, FAKE, ldw, qs.BF16, layout, 11008, FAKE, qs.F32,
                   FAKE, big, None)
    assert linear(11000) == 1                                 # ldw < n_out
    assert linear(11076) == 1                                 # ldw % 8
    assert linear(5000, layout=qs.LAYOUT_W) == 1              # pitched dense layout
    assert linear(1 << 17) == 2                               # W^T >= 1 GiB


def test_set_deterministic_returns_previous_setting():
    lib = qs.load()
    prev = lib.qs_set_deterministic(1)
    try:
        assert lib.qs_set_deterministic(0) == 1
        assert lib.qs_set_deterministic(7) == 0      # any nonzero value means on
        assert qs.qs_set_deterministic(False) is True
    finally:
        lib.qs_set_deterministic(prev)


def test_probe_library_is_separate():
    """The streaming-read probe the bench quotes bandwidth against lives in
    its own library: libqs.so does not export it."""
    lib = qs.load()
    assert not hasattr(lib, "qs_stream_read")
    probe = ctypes.CDLL(os.path.join(os.path.dirname(qs.lib_path()), "libqs_probe.so"))
    fn = probe.qsprobe_stream_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    assert fn(None, 1024, FAKE, None) == 1
    assert fn(FAKE, 1024, None, None) == 1
    assert fn(FAKE, 1000, FAKE, None) == 1                       # bytes % 16 != 0
    assert fn(ctypes.c_void_p(0x1008), 1024, FAKE, None) == 1    # misaligned
    assert fn(FAKE, 0, FAKE, None) == 0                          # nothing to read


def test_i8t_and_ffn_validation():
    lib = qs.load()
    need = qs.qs_workspace_bytes(qs.OP_SPARSE_LINEAR_I8T, 2, 256, 64)
    assert lib.qs_sparse_linear_i8t(FAKE, 2, 256, 10, FAKE, ctypes.c_float(1.0), 60, None,
                                    None, None, None, None, FAKE, need, None) == 2
    assert lib.qs_sparse_linear_i8t(FAKE, 2, 256, 257, FAKE, ctypes.c_float(1.0), 64, None,
                                    None, None, None, None, FAKE, need, None) == 1
    need = qs.qs_workspace_bytes(qs.OP_SPARSE_FFN_DRELU, 2, 256, 512)
    # dReLU needs bf16 and a gate; squared ReLU takes no gate
    assert lib.qs_sparse_ffn(FAKE, qs.F32, 2, 256, 512, qs.ACT_DRELU, 256, -1, FAKE, FAKE, FAKE,
                             None, None, FAKE, qs.F32, None, None, None, FAKE, need, None) == 2
    assert lib.qs_sparse_ffn(FAKE, qs.BF16, 2, 256, 512, qs.ACT_DRELU, 256, -1, None, FAKE, FAKE,
                             None, None, FAKE, qs.F32, None, None, None, FAKE, need, None) == 1
    need = qs.qs_workspace_bytes(qs.OP_SPARSE_FFN_RELU2, 2, 256, 512)
    assert lib.qs_sparse_ffn(FAKE, qs.BF16, 2, 256, 512, qs.ACT_RELU2, 100, 513, None, FAKE,
                             FAKE, None, None, FAKE, qs.F32, None, None, None, FAKE, need,
                             None) == 1
    assert lib.qs_sparse_ffn(FAKE, qs.BF16, 2, 256, 512, qs.ACT_RELU2, 100, 50, FAKE, FAKE,
                             FAKE, None, None, FAKE, qs.F32, None, None, None, FAKE, need,
                             None) == 1
    # gated squared ReLU: needs the gate, takes no biases; same workspace as squared ReLU
    assert qs.qs_workspace_bytes(qs.OP_SPARSE_FFN_RELU2_GLU, 2, 256, 512) == need
    assert lib.qs_sparse_ffn(FAKE, qs.BF16, 2, 256, 512, qs.ACT_RELU2_GLU, 100, 50, None, FAKE,
                             FAKE, None, None, FAKE, qs.F32, None, None, None, FAKE, need,
                             None) == 1
    assert lib.qs_sparse_ffn(FAKE, qs.BF16, 2, 256, 512, qs.ACT_RELU2_GLU, 100, 50, FAKE, FAKE,
                             FAKE, FAKE, None, FAKE, qs.F32, None, None, None, FAKE, need,
                             None) == 1
    assert lib.qs_sparse_ffn(FAKE, qs.BF16, 2, 256, 512, 3, 100, 50, FAKE, FAKE,
                             FAKE, None, None, FAKE, qs.F32, None, None, None, FAKE, need,
                             None) == 1


def test_workspace_sizes_depend_on_shape_only():
    for op in (qs.OP_SPARSE_LINEAR, qs.OP_SPARSE_LINEAR_I8T, qs.OP_SPARSE_FFN_RELU2,
               qs.OP_SPARSE_FFN_DRELU):
        a = qs.qs_workspace_bytes(op, 16, 4096, 11008)
        b = qs.qs_workspace_bytes(op, 16, 4096, 11008)
        assert a == b and a % 256 == 0
    assert qs.qs_workspace_bytes(qs.OP_TOPK_MASK, 16, 4096, 0) == 0
    with pytest.raises(qs.QSError):
        qs.qs_workspace_bytes(99, 1, 1, 1)


def test_ternarize_matches_oracle_bit_exactly():
    rng = np.random.default_rng(31)
    for shape in [(4, 8), (33, 64), (128, 96)]:
        w = rng.normal(0, 0.02, size=shape).astype(np.float32)
        w[0, 0] = 0.0
        t_lib, a_lib = qs.qs_ternarize(w)
        t_ref, a_ref = oracle.ternarize(w)
        assert np.float32(a_lib) == a_ref
        assert np.array_equal(t_lib, t_ref)


def test_ternarize_extreme_magnitudes():
    w = np.array([[1e-40, -3e38, 2.5e-3, 0.0], [7.0, -1e-45, 3e38, 1.0]], dtype=np.float32)
    t_lib, a_lib = qs.qs_ternarize(w)
    t_ref, a_ref = oracle.ternarize(w)
    assert np.float32(a_lib) == a_ref and np.array_equal(t_lib, t_ref)


def test_pack_ternary_roundtrip_through_oracle_decoder():
    rng = np.random.default_rng(37)
    t = rng.integers(-1, 2, size=(64, 40)).astype(np.int8)
    packed = qs.qs_pack_ternary(t)
    assert packed.shape == (40, 16)
    assert np.array_equal(oracle.unpack_ternary(packed, 64), t)
    with pytest.raises(qs.QSError):
        qs.qs_pack_ternary(np.full((4, 4), 2, dtype=np.int8))


def test_backward_validation_and_workspace():
    lib = qs.load()
    need = qs.qs_workspace_bytes(qs.OP_SPARSE_LINEAR_BACKWARD, 4, 1024, 512)
    assert need == 4 * 1024 * 2
    assert qs.qs_workspace_bytes(qs.OP_SPARSE_LINEAR_BACKWARD, 3, 8, 16) == 256

    def call(x=FAKE, xt=qs.BF16, rows=4, d=1024, k=100, w=FAKE, wt=qs.BF16, lay=qs.LAYOUT_W,
             n=512, dy=FAKE, dyt=qs.BF16, dx=FAKE, dxt=qs.F32, dw=FAKE, dwt=qs.F32, ws=None,
             wsb=0):
        return lib.qs_sparse_linear_backward(x, xt, rows, d, k, w, wt, lay, n, dy, dyt, dx, dxt,
                                             dw, dwt, ws, wsb, None)
    assert call(k=1025) == 1                         # k > d_in
    assert call(k=-1) == 1
    assert call(lay=5) == 1                          # unknown layout
    assert call(xt=qs.F32) == 2                      # bf16 only
    assert call(dyt=qs.F32) == 2
    assert call(dxt=qs.I8) == 2
    assert call(d=1020) == 2                         # d_in % 8
    assert call(n=500) == 2                          # n_out % 8
    assert call(rows=1 << 20, d=1024) == 2           # operand of 2^30 elements
    assert call(x=None) == 1
    assert call(w=None) == 1                         # w needed for dx
    assert call(dx=MISALIGNED) == 2
    assert call() == 3                               # dw without workspace
    assert call(ws=FAKE, wsb=need - 1) == 3
    assert call(dx=None, dw=None) == 0               # nothing asked: no-op


def test_block_sparse_validation_and_workspace():
    lib = qs.load()
    need = qs.qs_workspace_bytes(qs.OP_BLOCK_SPARSE_LINEAR, 5, 96, 64)
    # packed values: 2 slices x 5 rows x 64 B; positions: 2 slices x 3 chunks of 16 B
    assert need == ((2 * 5 * 64 + 255) // 256) * 256 + ((2 * 3 * 16 + 255) // 256) * 256

    def call(x=FAKE, xt=qs.BF16, rows=4, d=1024, w=FAKE, wt=qs.BF16, n=512, y=FAKE, yt=qs.F32,
             mask=None, ws=FAKE, wsb=None):
        wsb = qs.qs_workspace_bytes(qs.OP_BLOCK_SPARSE_LINEAR, rows, d, n) if wsb is None else wsb
        return lib.qs_block_sparse_linear(x, xt, rows, d, w, wt, n, y, yt, mask, ws, wsb, None)
    assert call(xt=qs.F32) == 2
    assert call(wt=qs.F32) == 2
    assert call(yt=qs.I8) == 2
    assert call(d=1000) == 2                          # d_in % 32
    assert call(n=500) == 2                           # n_out % 8
    assert call(d=0, wsb=1 << 20) == 1
    assert call(x=None) == 1
    assert call(mask=MISALIGNED) == 2
    assert call(wsb=16) == 3
    assert call(rows=0) == 0


def test_moe_validation_and_workspace():
    lib = qs.load()
    need = qs.qs_workspace_bytes(qs.OP_SPARSE_MOE_FFN, 2, 256, 512)
    assert need > 2 * 512 * 4 + 2 * 256 * 4

    def call(x=FAKE, dt=qs.BF16, rows=1, d=256, ffn=512, e=8, k=2, wr=FAKE, wg=FAKE, wu=FAKE,
             wd=FAKE, y=FAKE, yt=qs.F32, ws=FAKE, wsb=None):
        wsb = need if wsb is None else wsb
        return lib.qs_sparse_moe_ffn(x, dt, rows, d, ffn, e, k, wr, wg, wu, wd, None, None, y, yt,
                                     None, None, None, None, ws, wsb, None)
    assert call(k=9) == 1                            # top_k > n_experts
    assert call(k=0) == 1
    assert call(e=65, k=2) == 2                      # at most 64 experts
    assert call(dt=qs.F32) == 2
    assert call(d=8200) == 2                         # d <= 8192
    assert call(ffn=500) == 2                        # ffn % 8
    assert call(wr=None) == 1
    assert call(wsb=need - 1) == 3
    assert call(rows=0) == 0


def test_static_ffn_validation():
    """The allocation-free FFN rejects a shape whose workspace exceeds its
    per-GPU scratch before any HIP call, and rows == 0 is a no-op."""
    lib = qs.load()
    need = qs.qs_workspace_bytes(qs.OP_SPARSE_FFN_RELU2, 64, 4096, 11008)
    assert need > qs.STATIC_SCRATCH_BYTES
    assert qs.qs_workspace_bytes(qs.OP_SPARSE_FFN_RELU2, 16, 4096, 14336) <= qs.STATIC_SCRATCH_BYTES
    st = lib.qs_sparse_ffn_static(FAKE, qs.BF16, 64, 4096, 11008, qs.ACT_RELU2, 1638, 4403,
                                  None, FAKE, FAKE, None, None, FAKE, qs.F32, None, None, None,
                                  None)
    assert st == qs.QS_ERR_UNSUPPORTED and "scratch" in qs.qs_last_error()
    assert lib.qs_sparse_ffn_static(None, qs.BF16, 0, 4096, 11008, qs.ACT_RELU2, 1, 1, None,
                                    None, None, None, None, None, qs.F32, None, None, None,
                                    None) == qs.QS_OK
    assert lib.qs_sparse_ffn_static(FAKE, qs.BF16, 2, 4096, 11008, 9, 1, 1, None, FAKE, FAKE,
                                    None, None, FAKE, qs.F32, None, None, None, None) == 1
