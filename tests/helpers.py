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


# Below |ref| = 8 the bf16 spacing is at most 2^-5, so a correctly rounded output is within
# 2^-6 of the exact value and the flat bar leaves 2e-2 - 2^-6 for the arithmetic before
# the output rounding.  From 8 up, half an ulp (2^-5 and more) alone can exceed 2e-2; there
# the bound is that half ulp plus the same arithmetic allowance.
FLOOR_FROM = 8.0


def parity_bound(ref: np.ndarray, max_abs=BF16_MAX) -> np.ndarray:
    """Per-element max-abs bound: max_abs where |ref| < 8, else
    max(max_abs, half a bf16 ulp of ref + max_abs - 2^-6)."""
    big = np.maximum(max_abs, bf16_half_ulp(ref) + (max_abs - 2.0 ** -6))
    return np.where(np.abs(ref) < FLOOR_FROM, max_abs, big)


def assert_bf16_close(name: str, gpu: torch.Tensor, ref: np.ndarray, max_abs=BF16_MAX, mean_abs=BF16_MEAN):
    """The parity bar for a bf16 output, element by element:

        |gpu_i - ref_i| <= max_abs (2e-2)                          where |ref_i| < 8
        |gpu_i - ref_i| <= half a bf16 ulp of ref_i + max_abs - 2^-6  where |ref_i| >= 8
        mean_i |gpu_i - ref_i| <= mean_abs (2e-3)

    The message gives the error, the bf16 rounding floor max|bf16(ref) - ref|, and how
    many elements exceed the flat max_abs (only elements with |ref| >= 8 may)."""
    g = f64(gpu)
    err = np.abs(g - ref)
    bound = parity_bound(ref, max_abs)
    mx, mn = (float(err.max()), float(err.mean())) if err.size else (0.0, 0.0)
    n_flat = int((err > max_abs).sum())
    worst = float((err - bound).max()) if err.size else -1.0
    msg = (f"{name}: max_abs={mx:.3e} mean_abs={mn:.3e} bf16_floor={bf16_floor(ref):.3e} "
           f"max|ref|={np.abs(ref).max() if ref.size else 0.0:.3f} bar={max_abs:.1e} "
           f"over_flat_bar={n_flat}/{err.size} (|ref|>={FLOOR_FROM:g}: {int((np.abs(ref) >= FLOOR_FROM).sum())}) "
           f"worst_margin={-worst:.3e}")
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
