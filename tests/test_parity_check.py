"""CPU tests of the parity metrics themselves (tests/parity.py): the row
check must see a wrong late stretch of a long linear-attention output that
the slice check alone lets through."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import EPS, TOL, assert_parity, assert_rows, row_rel_err, slice_rel_err
from weight_recurrent_memory_amd import workloads as wl


@pytest.fixture(scope="module")
def long_la():
    # two heads of the bf16 prefill workload's shape (T = 8192, d = 64)
    q, k, v = wl.la_inputs(1, 2, 8192, 64, 64, torch.bfloat16, seed=2, device="cpu")
    o, _, _ = oracle.la_forward(q, k, v, eps=EPS)
    return o


def test_output_magnitude_falls_along_the_sequence(long_la):
    # the reason the slice check is not enough: |o_t| shrinks like a running mean
    n = np.linalg.norm(long_la[0, 0], axis=-1)
    assert n[:64].mean() > 10 * n[-1024:].mean()


@pytest.mark.parametrize("cut", [512, 2048])
def test_zeroed_tail_passes_the_slice_check_but_not_the_row_check(long_la, cut):
    x = long_la.copy()
    x[:, :, -cut:] = 0.0  # the last segment (or the last quarter) lost
    tol = TOL[torch.bfloat16]
    assert float(slice_rel_err(x, long_la, (2, 3)).max()) <= tol  # blind to it
    with pytest.raises(AssertionError, match="token-row error"):
        assert_rows(x, long_la, tol, "o")


def test_late_tokens_scaled_fail_the_row_check(long_la):
    x = long_la.copy()
    x[:, :, 6000:] *= 1.05  # 5 % off on the late tokens only
    with pytest.raises(AssertionError, match="token-row error"):
        assert_rows(x, long_la, TOL[torch.bfloat16], "o")


def test_rounding_noise_passes_both(long_la):
    rng = np.random.default_rng(0)
    x = long_la * (1 + 2.0 ** -8 * rng.standard_normal(long_la.shape))  # bf16-sized relative noise
    worst = assert_rows(x, long_la, TOL[torch.bfloat16], "o")
    assert worst < 1e-2


def test_row_error_closed_forms():
    r = np.array([[[[3.0, 4.0], [0.0, 0.0], [1.0, 0.0]]]])
    x = np.array([[[[3.0, 4.5], [0.0, 0.0], [1.0, 1.0]]]])
    e = row_rel_err(x, r)
    assert e.shape == (1, 1, 3)
    assert e[0, 0, 0] == pytest.approx(0.1)  # ||(0, .5)|| / ||(3, 4)||
    assert e[0, 0, 1] == 0.0                  # zero row matched exactly
    assert e[0, 0, 2] == pytest.approx(1.0)
    x2 = x.copy()
    x2[0, 0, 1, 0] = 1e-30                    # anything against a zero reference row fails
    assert np.isinf(row_rel_err(x2, r)[0, 0, 1])


def test_slice_check_unchanged_without_rows():
    r = np.ones((1, 2, 5, 3))
    x = r.copy()
    x[0, 1, 4, 2] = 1.01
    assert assert_parity(x, r, 2e-2, "o") == pytest.approx(0.01)
    with pytest.raises(AssertionError, match="slice error"):
        assert_parity(x, r, 1e-3, "o")


def test_row_floor_limits_only_small_rows():
    r = np.zeros((1, 1, 4, 2))
    r[0, 0, :, 0] = [1.0, 1.0, 1.0, 0.01]
    x = r.copy()
    x[0, 0, 3, 0] += 0.001  # 10 % of a row 100x below the median
    assert row_rel_err(x, r)[0, 0, 3] == pytest.approx(0.1)
    assert row_rel_err(x, r, floor=1 / 8)[0, 0, 3] == pytest.approx(0.008)
    x[0, 0, 1, 0] = 0.5     # a full-size row still fails at its own norm
    assert row_rel_err(x, r, floor=1 / 8)[0, 0, 1] == pytest.approx(0.5)
