"""GPU parity of Block Q-Sparse (qs_block_sparse_linear): the 2:4 block mask
is bit-exact against the oracle's block top-K on the bf16 magnitudes, and
y = (X (.) M) . W^T is within 4e-3 * T (bf16 products exact in fp32, fp32
sums, a bf16 output's rounding included), T = sum of |x_j w_j| over the kept
entries; integer-valued inputs are bit-exact."""
import numpy as np
import pytest

import datagen
import oracle
from gpu_util import assert_within, note, to_dev

pytestmark = pytest.mark.gpu


def _run(qs, x, w, ydt):
    import torch
    y, mask = qs.qs_block_sparse_linear(to_dev(x, torch.bfloat16), to_dev(w, torch.bfloat16),
                                        y_dtype=ydt, want_mask=True)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), mask.cpu().numpy()


def _ref(x, w):
    mask = oracle.block_topk_select(oracle.magnitude(x), 2, 4)
    y, t = oracle.sparse_linear(x, w, mask)
    return mask, y, t


@pytest.mark.parametrize("ydt", ["f32", "bf16"])
@pytest.mark.parametrize("rows,d,n", [(1, 32, 8), (5, 96, 40), (37, 256, 200), (300, 992, 136),
                                      (513, 128, 776), (256, 512, 384)])
def test_block_sparse_random(gpu_lib, ydt, rows, d, n):
    import torch
    qs = gpu_lib
    rng = np.random.default_rng(rows + 7 * d + n)
    x = datagen.bf16_round(datagen.student_t(rng, (rows, d)))
    w = datagen.bf16_round(datagen.normal(rng, (n, d), 0.02))
    note(f"block sparse rows={rows} d={d} n={n} y={ydt}")
    y, mask = _run(qs, x, w, torch.float32 if ydt == "f32" else torch.bfloat16)
    m_ref, y_ref, t = _ref(x, w)
    assert np.array_equal(mask, m_ref)
    assert_within(y, y_ref, t, 4e-3, "block sparse")


def test_block_sparse_ties_signs_and_zeros(gpu_lib):
    import torch
    qs = gpu_lib
    rng = np.random.default_rng(5)
    rows, d, n = 40, 128, 64
    x = rng.integers(-3, 4, size=(rows, d)).astype(np.float32)   # many ties inside blocks
    x[0] = 0.0                                                    # all-zero row
    x[1, :8] = [1.0, -1.0, 1.0, -1.0, 0.0, -0.0, 0.0, 2.0]        # x next to -x, signed zeros
    w = rng.integers(-2, 3, size=(n, d)).astype(np.float32)
    note("block sparse ties")
    y, mask = _run(qs, x, w, torch.float32)
    m_ref, y_ref, _ = _ref(x, w)
    assert np.array_equal(mask, m_ref)
    assert np.array_equal(y, y_ref)                               # integer-valued: exact
    assert np.all(mask.reshape(rows, -1, 4).sum(axis=2) == 2)


def test_block_sparse_full_c4_sampled(gpu_lib):
    """The fused-QKV prefill shape under Block Q-Sparse: X [2048, 4096],
    W [12288, 4096]; the mask is checked whole, y on 64 sampled rows."""
    import torch
    qs = gpu_lib
    c = datagen.c4_prefill_qkv()
    x, w = c["X"], c["W"]
    note("block sparse full C4")
    y, mask = _run(qs, x, w, torch.float32)
    m_ref = oracle.block_topk_select(oracle.magnitude(x), 2, 4)
    assert np.array_equal(mask, m_ref)
    rows = np.sort(np.random.default_rng(79).choice(x.shape[0], 64, replace=False))
    rows[0], rows[-1] = 0, x.shape[0] - 1
    y_ref, t = oracle.sparse_linear(x[rows], w, m_ref[rows])
    assert_within(y[rows], y_ref, t, 4e-3, "C4 block sparse")
