"""Shared helpers for the GPU parity tests (no arithmetic of the method)."""
import os

import numpy as np

REL_TOL = 2e-4   # |y - y_ref| <= 2e-4 * sum_c |w * x|, per output


def oracle_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_within_tolerance(y: np.ndarray, y_ref: np.ndarray, S: np.ndarray, what: str = ""):
    """Every output within REL_TOL * S of the f64 oracle; no NaN; S == 0
    requires y == +-0. Returns the largest |y - y_ref| / S."""
    y = np.asarray(y, np.float64)
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    assert not np.isnan(y).any(), f"{what}: NaN in output"
    err = np.abs(y - y_ref)
    bad = err > REL_TOL * S
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        raise AssertionError(
            f"{what}: {bad.sum()} outputs out of tolerance; first at flat index {i}: "
            f"y={y.ravel()[i]!r} ref={y_ref.ravel()[i]!r} S={S.ravel()[i]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(S > 0, err / S, 0.0)
    return float(rel.max()) if rel.size else 0.0


def sentinel_buffer(n: int, pad: int = 64):
    """A float32 device buffer of n + pad elements filled with a NaN pattern;
    the first n are the output, the pad must stay untouched."""
    import torch
    t = torch.full((n + pad,), float("nan"), dtype=torch.float32, device="cuda")
    return t


def assert_pad_untouched(t, n: int):
    tail = to_host(t)[n:]
    assert np.isnan(tail).all(), "a kernel wrote past the end of its output"
