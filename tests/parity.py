"""Parity helpers shared by the GPU tests.

Error metrics (the reading for the tolerance "relative error 1e-4 for fp32
inputs and 2e-2 for bf16 inputs"):

* slice check -- per (batch, head) slice (per (sequence, head, step) for
  decode): max|x - r| / max|r|, separately for o, S and z.  Elementwise
  relative error is meaningless here because outputs cross zero (values are
  zero-mean).
* row check -- for every output that has one row per token (o, the
  predictions, dq, dk, dv): per token t, ||x_t - r_t||_2 / ||r_t||_2, and its
  maximum over the tokens of each (batch, head).  The slice check alone is
  blind to most of a long sequence: a linear-attention output is a running
  weighted mean, so |o_t| falls from O(1) at the first tokens to about 0.01
  after a few thousand, and the slice maximum is set by the early tokens.
  Checking error against sequence length, at the real length, is what the
  Recurrence page ("手撕：递推与记忆模型", "验证边界") asks for.
"""
import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}

# The eps the kernels receive is the fp32 value of 1e-6; the oracle gets the
# same number, upcast.
EPS = float(np.float32(1e-6))


def to64(t):
    return t.detach().to("cpu").double().numpy()


def _arr(x):
    return to64(x) if isinstance(x, torch.Tensor) else np.asarray(x, dtype=np.float64)


def slice_rel_err(x, r, axes):
    """max over the non-slice axes of |x - r|, divided by max |r|, per slice."""
    x, r = np.asarray(x, dtype=np.float64), np.asarray(r, dtype=np.float64)
    num = np.abs(x - r).max(axis=axes)
    den = np.abs(r).max(axis=axes)
    return num / np.maximum(den, 1e-300)


def row_rel_err(x, r, floor=0.0):
    """||x_t - r_t|| / ||r_t|| for every row t (the last axis is the row).  A
    reference row of zeros must be matched by a row of zeros.  floor > 0
    divides instead by max(||r_t||, floor * median_t ||r_t||), the median over
    the rows of the same slice (all axes but the last two)."""
    x, r = np.asarray(x, dtype=np.float64), np.asarray(r, dtype=np.float64)
    num = np.sqrt(np.square(x - r).sum(axis=-1))
    den = np.sqrt(np.square(r).sum(axis=-1))
    if floor > 0 and den.ndim >= 1:
        den = np.maximum(den, floor * np.median(den, axis=-1, keepdims=True))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))


def assert_parity(x, r, tol, what, axes=None, rows=False, row_floor=0.0):
    """Slice check of x against the reference r; with rows=True also the row
    check (last axis = one token's row; row_floor as in row_rel_err).
    Returns the worst error found."""
    x, r = _arr(x), np.asarray(r, dtype=np.float64)
    assert x.shape == r.shape, (what, x.shape, r.shape)
    if axes is None:  # all axes after the first two are one slice
        axes = tuple(range(2, x.ndim))
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    err = slice_rel_err(x, r, axes)
    worst = float(np.max(err)) if err.size else 0.0
    assert worst <= tol, f"{what}: worst slice error {worst:.3e} > {tol:.1e}"
    if rows:
        rerr = row_rel_err(x, r, row_floor)
        if rerr.size:
            wr = float(np.max(rerr))
            if not wr <= tol:
                idx = np.unravel_index(int(np.argmax(rerr)), rerr.shape)
                raise AssertionError(f"{what}: worst token-row error {wr:.3e} > {tol:.1e} at index {idx}")
            worst = max(worst, wr)
    return worst


def assert_rows(x, r, tol, what):
    """Both checks for an output with one row per token ([..., T, d])."""
    return assert_parity(x, r, tol, what, rows=True)
