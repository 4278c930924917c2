"""Helpers for the GPU parity tests (device transfer, the attention tolerance)."""
import json
import os

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


# every comparison made by assert_attention_close in this process: what was
# compared, how many elements, and the achieved error (printed at the end of
# the run by tests/conftest.py, and appended as JSON lines to the file named by
# PA_PARITY_LOG if that is set)
MARGINS = []


def assert_attention_close(got, ref, what=""):
    """Elementwise |gpu - oracle| <= ATOL + RTOL * |oracle|.  Records the raw
    max-abs error, the max-rel error over elements with |oracle| >= ATOL / RTOL
    (= 0.2), and the largest |error| / (ATOL + RTOL |oracle|) (<= 1 passes)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    big = np.abs(ref) >= ATOL / RTOL
    rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    rec = {"case": what, "elements": int(got.size), "max_abs": float(err.max()) if err.size else 0.0,
           "max_rel_ref_ge_0.2": rel, "max_err_over_bound": float((err / bound).max()) if err.size else 0.0}
    MARGINS.append(rec)
    log = os.environ.get("PA_PARITY_LOG")
    if log:
        with open(log, "a") as fh:
            fh.write(json.dumps(rec) + "\n")
    excess = err - bound
    if excess.size and excess.max() > 0:
        i = np.unravel_index(np.argmax(excess), excess.shape)
        raise AssertionError(
            f"{what}: {int((excess > 0).sum())} elements out of tolerance; worst at {i}: "
            f"gpu={got[i]!r} oracle={ref[i]!r}; max-abs={rec['max_abs']:.3e} "
            f"max-rel(|ref|>=0.2)={rel:.3e}")
    return rec["max_abs"]


def bits16(a):
    return np.ascontiguousarray(a).view(np.uint16)
