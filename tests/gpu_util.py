"""Helpers for the GPU parity tests (device transfer, the attention tolerance)."""
import numpy as np
import torch

# attention outputs: |gpu - oracle| <= ATOL + RTOL * |oracle|, elementwise
ATOL = 2e-3
RTOL = 1e-2


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    return torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_attention_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    excess = np.abs(got - ref) - (ATOL + RTOL * np.abs(ref))
    if excess.max() > 0:
        i = np.unravel_index(np.argmax(excess), excess.shape)
        big = np.abs(ref) >= ATOL / RTOL
        rel = (np.abs(got - ref)[big] / np.abs(ref[big])).max() if big.any() else 0.0
        raise AssertionError(
            f"{what}: {int((excess > 0).sum())} elements out of tolerance; worst at {i}: "
            f"gpu={got[i]!r} oracle={ref[i]!r}; max-abs={np.abs(got - ref).max():.3e} "
            f"max-rel(|ref|>=0.2)={rel:.3e}")
    return float(np.abs(got - ref).max())


def bits16(a):
    return np.ascontiguousarray(a).view(np.uint16)
