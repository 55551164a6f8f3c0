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


def edge_max_abs(ref: np.ndarray, excess: float = 1e-2) -> float:
    """Max-abs bound for edge-shape tests: the 2e-2 bar, or, where bf16 output rounding
    alone already takes most of it (values of magnitude >= 4), that rounding floor plus
    ``excess`` of accumulated error.  The workload-config tests use the plain 2e-2 bar."""
    return max(BF16_MAX, bf16_floor(ref) + excess)


def assert_bf16_close(name: str, gpu: torch.Tensor, ref: np.ndarray, max_abs=BF16_MAX, mean_abs=BF16_MEAN):
    if max_abs == "edge":
        max_abs = edge_max_abs(ref)
    mx, mn = errors(gpu, ref)
    msg = (f"{name}: max_abs={mx:.3e} mean_abs={mn:.3e} bf16_floor={bf16_floor(ref):.3e} "
           f"max|ref|={np.abs(ref).max() if ref.size else 0.0:.3f} bound={max_abs:.3e}")
    print(msg, flush=True)
    assert np.isfinite(f64(gpu)).all(), name + ": non-finite values"
    assert mx <= max_abs and mn <= mean_abs, msg


def assert_lse_close(gpu: torch.Tensor, ref: np.ndarray, max_abs=LSE_MAX):
    mx, mn = errors(gpu, ref)
    msg = f"lse: max_abs={mx:.3e} mean_abs={mn:.3e}"
    print(msg, flush=True)
    assert np.isfinite(f64(gpu)).all(), "lse: non-finite values"
    assert mx <= max_abs, msg


def gpu_available() -> bool:
    return torch.cuda.is_available()
