"""The softmax's exp2: the cubic polynomial on the host (CPU) and both device forms (GPU)."""

import numpy as np
import pytest
import torch

import exact_attention_27_amd as ea

GRID = np.concatenate([np.linspace(-126.0, 30.0, 400001), np.arange(-126, 31, dtype=np.float64)]).astype(np.float32)


def rel_err(y, x):
    ref = np.exp2(x.astype(np.float64))
    return np.abs(y.astype(np.float64) - ref) / ref


def test_poly_relative_error_bound():
    """Max relative error of the degree-3 polynomial over normal results, against fp64 2^x."""
    y = ea.attn_exp2_poly_host(GRID)
    err = rel_err(y, GRID)
    assert err.max() <= 1.2e-4, err.max()
    assert err.max() >= 5e-5  # a cubic cannot do much better: catches a silently swapped-in exact exp


def test_poly_special_values():
    x = np.array([0.0, -np.inf, -127.0, -1000.0, 1.0, 8.0, -1.0], dtype=np.float32)
    y = ea.attn_exp2_poly_host(x)
    assert y[0] == 1.0
    assert y[1] == 0.0 and y[2] == 0.0 and y[3] == 0.0
    assert y[4] == 2.0 and y[5] == 256.0 and y[6] == 0.5  # integers are exact: p(0) = 1


def test_poly_large_arguments_saturate():
    """Arguments above 64 (up to +inf) give 2^64: large enough for the forward's rescale
    test, which sees a tile's exponentials before deciding to rescale."""
    x = np.array([64.0, 64.5, 100.0, 127.0, 128.0, 200.0, 1000.0, 1e30, np.inf], dtype=np.float32)
    y = ea.attn_exp2_poly_host(x)
    assert (y == 2.0 ** 64).all(), y


def test_poly_tiny_results_are_tiny():
    x = np.linspace(-127.0, -125.0, 2001).astype(np.float32)
    y = ea.attn_exp2_poly_host(x)
    assert (y >= 0).all() and (y <= 2.0 ** -124).all()


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [ea.ATTN_EXP_HW, ea.ATTN_EXP_POLY3])
def test_device_exp2(mode):
    x = torch.from_numpy(np.concatenate([GRID, np.array([-np.inf, -200.0, 0.0], dtype=np.float32)])).cuda()
    y = ea.attn_exp2_eval(x, mode).cpu().numpy()
    xs = x.cpu().numpy()
    n = GRID.size
    if mode == ea.ATTN_EXP_POLY3:
        np.testing.assert_array_equal(y, ea.attn_exp2_poly_host(xs))  # same arithmetic on both sides
        assert rel_err(y[:n], xs[:n]).max() <= 1.2e-4
    else:
        assert rel_err(y[:n], xs[:n]).max() <= 2e-6
    assert y[n] == 0.0 and y[n + 1] == 0.0 and y[n + 2] == 1.0
