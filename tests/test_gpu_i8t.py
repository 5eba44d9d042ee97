"""GPU parity of the quantised path (int8 absmax activations x packed ternary
weights): q, s, the index list, the int32 accumulators and the dequantised
output must all match the oracle bit for bit.  The weights are prepared by
the library's host routines (qs_ternarize / qs_pack_ternary) and, for the
oracle, by its own ternarize."""
import numpy as np
import pytest

import datagen
import oracle
from gpu_util import note, to_dev

pytestmark = pytest.mark.gpu


def _case(gpu_lib, x, w, k):
    import torch
    qs = gpu_lib
    n, d = w.shape
    t_lib, alpha = qs.qs_ternarize(w)
    packed = qs.qs_pack_ternary(t_lib)
    acc, y, xq, xs, idx = qs.qs_sparse_linear_i8t(to_dev(x), k, to_dev(packed), alpha, n)
    torch.cuda.synchronize()
    acc, y, xq, xs, idx = (a.cpu().numpy() for a in (acc, y, xq, xs, idx))

    q_ref, s_ref, _ = oracle.absmax_quant_i8(x)
    t_ref, a_ref = oracle.ternarize(w)
    m_ref, i_ref, _, _ = oracle.topk_select(oracle.magnitude(q_ref), k)
    acc_ref, y_ref = oracle.i8t_linear(q_ref, s_ref, t_ref, a_ref, m_ref)
    assert np.float32(alpha) == a_ref
    assert np.array_equal(xq, q_ref)
    assert np.array_equal(xs.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(idx, i_ref)
    assert np.array_equal(acc, acc_ref)
    assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))


@pytest.mark.parametrize("rows,d,n", [(1, 64, 16), (3, 300, 48), (5, 1000, 1040),
                                      # 1-4 tokens: the one-launch kernel (ragged column
                                      # tiles, runs past the row end, d % 4 != 0 elsewhere)
                                      (2, 64, 16), (4, 4096, 48), (3, 1000, 1040), (1, 301, 32),
                                      (9, 513, 2064), (33, 256, 64),
                                      # token batches: the int8 matrix-core kernel (ragged
                                      # feature steps, column tiles and token tiles)
                                      (16, 64, 16), (64, 1040, 400), (100, 512, 272),
                                      (130, 2048, 128)])
def test_i8t_random(gpu_lib, rows, d, n):
    rng = np.random.default_rng(rows + d + n)
    x = datagen.student_t(rng, (rows, d))
    w = datagen.normal(rng, (n, d), 0.02)
    for k in sorted({0, 1, (31 * d) // 80, d}):
        note(f"i8t rows={rows} d={d} n={n} k={k}")
        _case(gpu_lib, x, w, k)


def test_i8t_special_rows(gpu_lib):
    rng = np.random.default_rng(53)
    x = np.zeros((4, 256), dtype=np.float32)
    x[1] = -1.25                        # constant row: q = -127 everywhere, first K
    x[2, 17] = 3.0                      # one-hot
    x[3] = datagen.student_t(rng, (256,)) * 1e-7    # tiny magnitudes: eps matters
    w = datagen.normal(rng, (32, 256), 0.02)
    for k in (0, 5, 99, 256):
        note(f"i8t special rows k={k}")
        _case(gpu_lib, x, w, k)


@pytest.mark.parametrize("batch", [1, 4, 16, 64])
def test_i8t_full_c3(gpu_lib, batch):
    c = datagen.c3_i8t_linear(batch)
    note(f"i8t full config C3 B={batch}")
    _case(gpu_lib, c["X"], c["W"], c["K"])


@pytest.mark.parametrize("batch", [1, 2, 4])
def test_i8t_bench_call(gpu_lib, batch):
    """The call the benchmark times: acc and y only (no q, s or index list)."""
    import torch
    qs = gpu_lib
    c = datagen.c3_i8t_linear(batch)
    n, d = c["W"].shape
    t_lib, alpha = qs.qs_ternarize(c["W"])
    packed = to_dev(qs.qs_pack_ternary(t_lib))
    acc = torch.empty((batch, n), dtype=torch.int32, device="cuda")
    y = torch.empty((batch, n), dtype=torch.float32, device="cuda")
    note(f"i8t bench call C3 B={batch}")
    qs.qs_sparse_linear_i8t(to_dev(c["X"]), c["K"], packed, alpha, n, acc=acc, y=y, want_all=False)
    torch.cuda.synchronize()
    q_ref, s_ref, _ = oracle.absmax_quant_i8(c["X"])
    t_ref, a_ref = oracle.ternarize(c["W"])
    m_ref, _, _, _ = oracle.topk_select(oracle.magnitude(q_ref), c["K"])
    acc_ref, y_ref = oracle.i8t_linear(q_ref, s_ref, t_ref, a_ref, m_ref)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))
