"""Helpers for the GPU parity tests (marshalling and tolerance checks)."""
import sys

import numpy as np


def note(msg: str):
    """Name the case before a GPU step, flushed, so a fault can be attributed."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    if dtype is not None:
        t = t.to(dtype)
    return t


def key_bits(tau_mag: np.ndarray, kind: str) -> np.ndarray:
    """Magnitudes (from the oracle) -> the library's u32 key bits."""
    tau_mag = np.asarray(tau_mag, dtype=np.float64)
    out = np.full(tau_mag.shape, 0xFFFFFFFF, dtype=np.uint32)
    fin = np.isfinite(tau_mag)
    if kind == "f32":
        out[fin] = tau_mag[fin].astype(np.float32).view(np.uint32) & 0x7FFFFFFF
    elif kind == "bf16":
        out[fin] = (tau_mag[fin].astype(np.float32).view(np.uint32) >> 16) & 0x7FFF
    elif kind == "i8":
        out[fin] = tau_mag[fin].astype(np.uint32)
    else:
        raise ValueError(kind)
    return out


def assert_within(y, y_ref, t, tol, what=""):
    """|y - y_ref| <= tol * T elementwise; T == 0 requires y == 0."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    bound = tol * t
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), y.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {y.size} outside tol*T; worst at {i}: "
            f"y={y[i]!r} ref={y_ref[i]!r} T={t[i]!r} tol={tol}")
    zero = t == 0
    assert np.all(y[zero] == 0), f"{what}: nonzero output where T == 0"
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(t > 0, err / t, 0.0)
    return float(rel.max()) if rel.size else 0.0


class reduction_mode:
    """Context manager: fixed-order (deterministic=True) or atomic split-K sums."""

    def __init__(self, qs, deterministic: bool):
        self.qs, self.det, self.prev = qs, deterministic, None

    def __enter__(self):
        self.prev = self.qs.qs_set_deterministic(self.det)
        return self

    def __exit__(self, *exc):
        self.qs.qs_set_deterministic(self.prev)
        return False
