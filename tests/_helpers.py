"""Shared test helpers: tolerance check and device upload."""
import numpy as np

# fp32 outputs: pass iff |gpu - oracle| <= max(2e-3 * |oracle|, 1e-4) elementwise.
REL_TOL = 2e-3
ABS_TOL = 1e-4


def assert_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), what + ": non-finite output"
    err = np.abs(gpu - ref)
    tol = np.maximum(REL_TOL * np.abs(ref), ABS_TOL)
    bad = err > tol
    if bad.any():
        i = np.flatnonzero(bad.ravel())[:5]
        raise AssertionError("%s: %d/%d elements out of tolerance; first %s gpu=%s ref=%s"
                             % (what, bad.sum(), bad.size, i.tolist(), gpu.ravel()[i].tolist(),
                                ref.ravel()[i].tolist()))
    return float((err / np.maximum(np.abs(ref), ABS_TOL / REL_TOL)).max()) if err.size else 0.0


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")
