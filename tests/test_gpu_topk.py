"""GPU parity of the top-K selection kernel against the oracle: masks, index
lists and (tau, cutoff) descriptors must match bit for bit."""
import numpy as np
import pytest

import datagen
import oracle
from gpu_util import key_bits, note, to_dev

pytestmark = pytest.mark.gpu


def _inputs(kind, rows, d, seed, ties):
    rng = np.random.default_rng(seed)
    if kind == "i8":
        x = rng.integers(-128, 128, size=(rows, d)).astype(np.int8)
        if ties:
            x = (x // 16).astype(np.int8)
        return x
    x = datagen.student_t(rng, (rows, d))
    if ties:
        x = (np.round(x * 4) / 4).astype(np.float32)
        x[:, 1::2] = -x[:, 0::2][:, : d // 2]          # exact x / -x pairs
    if kind == "bf16":
        x = datagen.bf16_round(x)
    return x


def _run(gpu_lib, kind, x, k):
    import torch
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8}[kind]
    xd = to_dev(x, dt)
    mask, idx, tau, cut = gpu_lib.qs_topk_mask(xd, k)
    torch.cuda.synchronize()
    return (mask.cpu().numpy(), idx.cpu().numpy(), tau.cpu().numpy().view(np.uint32),
            cut.cpu().numpy())


def _check(kind, x, k, got):
    mask, idx, tau, cut = got
    m_ref, i_ref, t_ref, c_ref = oracle.topk_select(oracle.magnitude(x.astype(np.float64)), k)
    assert np.array_equal(mask, m_ref)
    assert np.array_equal(idx, i_ref)
    assert np.array_equal(tau, key_bits(t_ref, kind))
    assert np.array_equal(cut, c_ref)


@pytest.mark.parametrize("kind", ["f32", "bf16", "i8"])
@pytest.mark.parametrize("rows,d", [(1, 1), (3, 7), (2, 64), (5, 1000), (1, 4096), (70, 300),
                                    (2, 14336), (2, 20000)])
@pytest.mark.parametrize("ties", [False, True])
def test_topk_parity(gpu_lib, kind, rows, d, ties):
    x = _inputs(kind, rows, d, seed=rows * 1000 + d + ties, ties=ties)
    for k in sorted({0, 1, d // 3, d // 2, d - 1, d} - {-1}):
        if k < 0:
            continue
        note(f"topk {kind} rows={rows} d={d} k={k} ties={ties}")
        _check(kind, x, k, _run(gpu_lib, kind, x, k))


def test_topk_special_rows(gpu_lib):
    x = np.zeros((6, 513), dtype=np.float32)
    x[1] = 2.5                          # constant: first K
    x[2, ::2] = -1.0                    # x next to -x
    x[2, 1::2] = 1.0
    x[3] = -0.0                         # all negative zero
    x[4, 100] = 7.0                     # one-hot
    x[5] = np.arange(513, dtype=np.float32)[::-1]
    for k in (0, 1, 50, 512, 513):
        note(f"topk special rows k={k}")
        _check("f32", x, k, _run(gpu_lib, "f32", x, k))


@pytest.mark.parametrize("cfg", ["c1", "c2", "c4"])
def test_topk_full_configs(gpu_lib, cfg):
    if cfg == "c1":
        c = datagen.c1_linear(with_weights=False)
        x, k, kind = c["X"], c["K"], "f32"
    elif cfg == "c2":
        c = datagen.c2_relu2_ffn(16, with_weights=False)
        x, k, kind = c["X"], c["K_in"], "bf16"
    else:
        c = datagen.c4_prefill_qkv(with_weights=False)
        x, k, kind = c["X"], c["K"], "bf16"
    note(f"topk full config {cfg} shape={x.shape} k={k}")
    _check(kind, x, k, _run(gpu_lib, kind, x, k))


@pytest.mark.parametrize("nbin", [20, 64, 65, 128, 200, 256, 257, 600])
def test_topk_boundary_bin_sizes(gpu_lib, nbin):
    """fp32 rows whose threshold falls among nbin keys that share their top
    12 bits (1 + i 2^-20 differ only in low mantissa bits), some of them
    tied, so the select's last digits run over 1 to 4 register slots per lane
    (nbin <= 256) or over its LDS histograms (more)."""
    rng = np.random.default_rng(7000 + nbin)
    d = 4096
    big = 1200
    x = np.full(d, 1e-3, dtype=np.float32)
    x[:big] = 8.0 + rng.random(big).astype(np.float32)
    i = rng.integers(0, 40, size=nbin)                    # values repeat: ties in the bin
    x[big:big + nbin] = (1.0 + i * 2.0 ** -20).astype(np.float32)
    x *= np.where(rng.random(d) < 0.5, -1.0, 1.0).astype(np.float32)
    x = x[rng.permutation(d)][None, :].copy()
    for k in sorted({big + 1, big + nbin // 3, big + nbin // 2, big + nbin - 1, big + nbin}):
        note(f"topk boundary bin nbin={nbin} k={k}")
        _check("f32", x, k, _run(gpu_lib, "f32", x, k))


@pytest.mark.parametrize("rows,d", [(1, 8), (2, 4096), (3, 1000), (4, 4104), (2, 8192), (64, 512),
                                    (2, 8200), (5, 1004), (65, 520)])
@pytest.mark.parametrize("ties", [False, True])
def test_topk_xs_only_bf16(gpu_lib, rows, d, ties):
    """bf16 rows whose only output is X (.) M in fp32 (the decode FFN's
    selection launch): a selected entry is the bf16 value widened exactly, an
    unselected one +0.0, bit for bit; d % 8 == 0 with d <= 8192 and at most
    64 rows take the lean two-level kernel, the other shapes the general one."""
    import torch
    x = _inputs("bf16", rows, d, seed=5000 + rows * 7 + d + ties, ties=ties)
    xd = to_dev(x, torch.bfloat16)
    for k in sorted({0, 1, d // 3, d // 2, d - 1, d}):
        note(f"topk xs-only bf16 rows={rows} d={d} k={k} ties={ties}")
        got = gpu_lib.qs_topk_mask(xd, k, want_mask=False, want_idx=False, want_desc=False,
                                   want_xs=True)[4]
        torch.cuda.synchronize()
        m_ref = oracle.topk_select(oracle.magnitude(x.astype(np.float64)), k)[0].astype(bool)
        ref = np.where(m_ref, x.astype(np.float32), np.float32(0.0)).astype(np.float32)
        assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))
