"""Parity helpers shared by the GPU tests.

Error metric (the reading for the tolerance "relative error 1e-4 for fp32
inputs and 2e-2 for bf16 inputs"): per (batch, head) slice -- per (sequence,
head, step) for decode -- max|x - r| / max|r|, computed separately for o, S
and z.  Elementwise relative error is meaningless here because outputs cross
zero (values are zero-mean).
"""
import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}

# The eps the kernels receive is the fp32 value of 1e-6; the oracle gets the
# same number, upcast.
EPS = float(np.float32(1e-6))


def to64(t):
    return t.detach().to("cpu").double().numpy()


def slice_rel_err(x, r, axes):
    """max over the non-slice axes of |x - r|, divided by max |r|, per slice."""
    x, r = np.asarray(x, dtype=np.float64), np.asarray(r, dtype=np.float64)
    num = np.abs(x - r).max(axis=axes)
    den = np.abs(r).max(axis=axes)
    return num / np.maximum(den, 1e-300)


def assert_parity(x, r, tol, what, axes=None):
    x = to64(x) if isinstance(x, torch.Tensor) else np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert x.shape == r.shape, (what, x.shape, r.shape)
    if axes is None:  # all axes after the first two are one slice
        axes = tuple(range(2, x.ndim))
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    err = slice_rel_err(x, r, axes)
    worst = float(np.max(err))
    assert worst <= tol, f"{what}: worst slice error {worst:.3e} > {tol:.1e}"
    return worst
