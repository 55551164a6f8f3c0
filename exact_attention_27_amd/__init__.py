"""Python binding of libattn.so, the gfx950 exact-attention library (C ABI in include/attn.h).

Argument marshalling only: every step of the computation runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  There is no fallback:
if libattn.so is missing or fails to load, every call raises.

The functions carry the C names:
    attn_fwd, attn_fwd_ex, attn_fwd_varlen, attn_bwd, attn_bwd_ex, attn_bwd_phase, attn_bwd_workspace_bytes,
    attn_bwd_noalloc, attn_launch_plan, attn_default_options, attn_status_string, attn_exp2_eval,
    attn_exp2_poly_host
and `attention` joins attn_fwd and attn_bwd under torch autograd.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "AttnError", "attn_options", "library_path", "lib",
    "attn_fwd", "attn_fwd_ex", "attn_fwd_varlen", "attn_bwd", "attn_bwd_ex", "attn_bwd_phase", "attn_bwd_workspace_bytes",
    "attn_bwd_varlen", "attn_bwd_varlen_workspace_bytes",
    "attn_bwd_noalloc", "ATTN_ERR_SCRATCH", "attn_launch_plan", "attn_plan", "attention", "attention_varlen",
    "attn_default_options", "attn_status_string", "attn_exp2_eval", "attn_exp2_poly_host",
    "ATTN_EXP_HW", "ATTN_EXP_POLY3", "ATTN_VARIANT_AUTO", "ATTN_VARIANT_PINGPONG", "ATTN_VARIANT_FOURWAVE",
]

ATTN_EXP_HW = 0
ATTN_EXP_POLY3 = 1
ATTN_VARIANT_AUTO = 0
ATTN_VARIANT_PINGPONG = 1
ATTN_VARIANT_FOURWAVE = 2

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libattn.so")


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class attn_options(ctypes.Structure):
    _fields_ = [("exp_mode", ctypes.c_int), ("tau", ctypes.c_float), ("variant", ctypes.c_int)]


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float


class attn_plan(ctypes.Structure):
    _fields_ = [("fwd_schedule", ctypes.c_int), ("fwd_chunk", ctypes.c_int), ("dq_chunk", ctypes.c_int),
                ("dkdv_chunk", ctypes.c_int), ("dkdv_schedule", ctypes.c_int)]


def lib() -> ctypes.CDLL:
    """The loaded libattn.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(python -m exact_attention_27_amd.build)")
        L = ctypes.CDLL(path)
        L.attn_default_options.restype = attn_options
        L.attn_default_options.argtypes = []
        L.attn_status_string.restype = ctypes.c_char_p
        L.attn_status_string.argtypes = [_I]
        L.attn_fwd.restype = _I
        L.attn_fwd.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]
        L.attn_fwd_varlen.restype = _I
        L.attn_fwd_varlen.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I,
                                      ctypes.POINTER(attn_options), _P]
        L.attn_fwd_ex.restype = _I
        L.attn_fwd_ex.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I,
                                  ctypes.POINTER(attn_options), _P]
        L.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.attn_bwd_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
        L.attn_bwd.restype = _I
        L.attn_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I,
                               _P, ctypes.c_size_t, _P]
        L.attn_bwd_ex.restype = _I
        L.attn_bwd_ex.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I,
                                  _P, ctypes.c_size_t, ctypes.POINTER(attn_options), _P]
        L.attn_bwd_phase.restype = _I
        L.attn_bwd_phase.argtypes = [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I,
                                     _P, ctypes.c_size_t, ctypes.POINTER(attn_options), _P]
        L.attn_bwd_varlen_workspace_bytes.restype = ctypes.c_size_t
        L.attn_bwd_varlen_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
        L.attn_bwd_varlen.restype = _I
        L.attn_bwd_varlen.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I,
                                      _P, ctypes.c_size_t, ctypes.POINTER(attn_options), _P]
        L.attn_bwd_noalloc.restype = _I
        L.attn_bwd_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]
        L.attn_exp2_eval.restype = _I
        L.attn_exp2_eval.argtypes = [_P, _P, ctypes.c_long, _I, _P]
        L.attn_launch_plan.restype = _I
        L.attn_launch_plan.argtypes = [_I, _I, _I, _I, _I, _I, ctypes.POINTER(attn_options), ctypes.POINTER(attn_plan)]
        L.attn_exp2_poly_host.restype = None
        L.attn_exp2_poly_host.argtypes = [_P, _P, ctypes.c_long]
        _lib = L
    return _lib


def attn_status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def attn_default_options() -> attn_options:
    return lib().attn_default_options()


def _check(status: int) -> None:
    if status != 0:
        raise AttnError(status, attn_status_string(status))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class _Nothing:
    def __enter__(self):
        return None

    def __exit__(self, *exc):
        return False


_NOTHING = _Nothing()


def _on(device: torch.device):
    """torch.cuda.device(device), or nothing when it is already the current device (the
    context manager costs microseconds per call, which short launches feel)."""
    if device.type == "cuda" and device.index is not None and device.index == torch.cuda.current_device():
        return _NOTHING
    return torch.cuda.device(device)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream))


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape) -> None:
    """Type, dtype, shape and layout of one operand (the device is checked by _same_gpu)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_gpu(**tensors) -> None:
    """Every operand on one GPU device (the first one's)."""
    device = None
    for name, t in tensors.items():
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device (got {t.device})")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{name} is on {t.device}, the other operands on {device}")


def _options(opt, exp_mode, tau, variant=None):
    if opt is None and exp_mode is None and tau is None and variant is None:
        return None
    o = attn_default_options() if opt is None else attn_options(opt.exp_mode, opt.tau, opt.variant)
    if exp_mode is not None:
        o.exp_mode = int(exp_mode)
    if tau is not None:
        o.tau = float(tau)
    if variant is not None:
        o.variant = int(variant)
    return o


def _dims(q: torch.Tensor, k: torch.Tensor):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B,Hq,S,d] and k, v [B,Hkv,S,d]")
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    return B, Hq, Hkv, S, d


def attn_fwd_ex(q, k, v, scale: Optional[float] = None, causal: bool = False,
                o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                opt: Optional[attn_options] = None, exp_mode: Optional[int] = None,
                tau: Optional[float] = None, stream=None, variant: Optional[int] = None
                ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward pass; returns (o [B,Hq,S,d] bf16, lse [B,Hq,S] fp32).  scale defaults to 1/sqrt(d).
    variant: ATTN_VARIANT_AUTO (default), ATTN_VARIANT_PINGPONG or ATTN_VARIANT_FOURWAVE (the
    forward schedule; they round differently, each within the stated accuracy)."""
    B, Hq, Hkv, S, d = _dims(q, k)
    _need(q, "q", torch.bfloat16, (B, Hq, S, d))
    _need(k, "k", torch.bfloat16, (B, Hkv, S, d))
    _need(v, "v", torch.bfloat16, (B, Hkv, S, d))
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.bfloat16, (B, Hq, S, d))
    _need(lse, "lse", torch.float32, (B, Hq, S))
    _same_gpu(q=q, k=k, v=v, o=o, lse=lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    op = _options(opt, exp_mode, tau, variant)
    with _on(q.device):
        st = lib().attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, S, d,
                               scale, int(bool(causal)), None if op is None else ctypes.byref(op),
                               _stream(stream))
    _check(st)
    return o, lse


def attn_fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, scale: Optional[float] = None, causal: bool = False,
                    o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    opt: Optional[attn_options] = None, exp_mode: Optional[int] = None,
                    tau: Optional[float] = None, stream=None, variant: Optional[int] = None
                    ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward pass over a packed batch of sequences of different lengths.

    q: [total, Hq, d], k and v: [total, Hkv, d] bf16; cu_seqlens: [nseq + 1] int32 device
    tensor of token offsets; max_seqlen should be >= every length (query rows past it
    are not written).  Returns (o [total, Hq, d] bf16, lse [Hq, total] fp32).  scale
    defaults to 1/sqrt(d)."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q and k must be [total, H, d]")
    total, Hq, d = (int(x) for x in q.shape)
    Hkv = int(k.shape[1])
    _need(q, "q", torch.bfloat16, (total, Hq, d))
    _need(k, "k", torch.bfloat16, (total, Hkv, d))
    _need(v, "v", torch.bfloat16, (total, Hkv, d))
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor")
    nseq = int(cu_seqlens.numel()) - 1
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Hq, total), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.bfloat16, (total, Hq, d))
    _need(lse, "lse", torch.float32, (Hq, total))
    _same_gpu(q=q, k=k, v=v, cu_seqlens=cu_seqlens, o=o, lse=lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    op = _options(opt, exp_mode, tau, variant)
    with _on(q.device):
        st = lib().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens),
                                   max(nseq, 0), total, int(max_seqlen), Hq, Hkv, d, scale, int(bool(causal)),
                                   None if op is None else ctypes.byref(op), _stream(stream))
    _check(st)
    return o, lse


def attn_bwd_varlen(q, k, v, o, lse, do, cu_seqlens, max_seqlen: int, scale: Optional[float] = None,
                    causal: bool = False, dq=None, dk=None, dv=None, workspace: Optional[torch.Tensor] = None,
                    opt: Optional[attn_options] = None, exp_mode: Optional[int] = None,
                    tau: Optional[float] = None, stream=None, variant: Optional[int] = None):
    """Backward pass over a packed batch (the gradients of attn_fwd_varlen).

    q, o, do: [total, Hq, d], k and v: [total, Hkv, d] bf16; lse: [Hq, total] fp32 (as
    attn_fwd_varlen returns it); cu_seqlens: [nseq + 1] int32 device tensor of token
    offsets; max_seqlen must be >= every length.  Returns (dq, dk, dv) in the layouts of
    q, k and v; rows outside every sequence are left as allocated (torch.empty).
    workspace (uint8, >= attn_bwd_varlen_workspace_bytes(nseq, total, Hq, Hkv, d)) is
    allocated with torch when not given.  scale defaults to 1/sqrt(d)."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q and k must be [total, H, d]")
    total, Hq, d = (int(x) for x in q.shape)
    Hkv = int(k.shape[1])
    _need(q, "q", torch.bfloat16, (total, Hq, d))
    _need(k, "k", torch.bfloat16, (total, Hkv, d))
    _need(v, "v", torch.bfloat16, (total, Hkv, d))
    _need(o, "o", torch.bfloat16, (total, Hq, d))
    _need(lse, "lse", torch.float32, (Hq, total))
    _need(do, "do", torch.bfloat16, (total, Hq, d))
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor")
    nseq = max(int(cu_seqlens.numel()) - 1, 0)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", torch.bfloat16, (total, Hq, d))
    _need(dk, "dk", torch.bfloat16, (total, Hkv, d))
    _need(dv, "dv", torch.bfloat16, (total, Hkv, d))
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor")
    _same_gpu(q=q, k=k, v=v, o=o, lse=lse, do=do, cu_seqlens=cu_seqlens, dq=dq, dk=dk, dv=dv,
              **({} if workspace is None else {"workspace": workspace}))
    nbytes = attn_bwd_varlen_workspace_bytes(nseq, total, Hq, Hkv, d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    op = _options(opt, exp_mode, tau, variant)
    with _on(q.device):
        st = lib().attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens), nseq, total, int(max_seqlen),
                                   Hq, Hkv, d, scale, int(bool(causal)), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   None if op is None else ctypes.byref(op), _stream(stream))
    _check(st)
    return dq, dk, dv


def attn_fwd(q, k, v, scale: Optional[float] = None, causal: bool = False,
             o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None):
    """Forward pass with the default options (see attn_fwd_ex)."""
    return attn_fwd_ex(q, k, v, scale, causal, o, lse, stream=stream)


def attn_launch_plan(B: int, Hq: int, Hkv: int, S: int, d: int, causal: bool = False,
                     opt: Optional[attn_options] = None, *, exp_mode: Optional[int] = None,
                     tau: Optional[float] = None, variant: Optional[int] = None) -> dict:
    """The launch plan (schedules and dispatch chunks) of attn_launch_plan, as a dict."""
    op = _options(opt, exp_mode, tau, variant)
    out = attn_plan()
    _check(lib().attn_launch_plan(B, Hq, Hkv, S, d, int(bool(causal)), ctypes.byref(op) if op is not None else None,
                                  ctypes.byref(out)))
    return {n: getattr(out, n) for n, _ in attn_plan._fields_}


def attn_bwd_workspace_bytes(B: int, Hq: int, Hkv: int, S: int, d: int) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, Hq, Hkv, S, d))


def attn_bwd_varlen_workspace_bytes(nseq: int, total: int, Hq: int, Hkv: int, d: int) -> int:
    return int(lib().attn_bwd_varlen_workspace_bytes(nseq, total, Hq, Hkv, d))


ATTN_BWD_ALL, ATTN_BWD_PREPROCESS, ATTN_BWD_MAIN, ATTN_BWD_DQ = 0, 1, 2, 3


def attn_bwd_ex(q, k, v, o, lse, do, scale: Optional[float] = None, causal: bool = False,
                dq=None, dk=None, dv=None, workspace: Optional[torch.Tensor] = None,
                opt: Optional[attn_options] = None, exp_mode: Optional[int] = None,
                tau: Optional[float] = None, stream=None, variant: Optional[int] = None):
    """Backward pass; returns (dq, dk, dv).  workspace (uint8, >= attn_bwd_workspace_bytes)
    is allocated with torch when not given.  variant: the dK/dV kernel's schedule
    (ATTN_VARIANT_AUTO, ATTN_VARIANT_PINGPONG for eight-wave workgroups, ATTN_VARIANT_FOURWAVE
    for four-wave ones)."""
    return attn_bwd_phase(ATTN_BWD_ALL, q, k, v, o, lse, do, scale, causal, dq, dk, dv, workspace,
                          opt, exp_mode, tau, stream, variant)


def attn_bwd_phase(phase: int, q, k, v, o, lse, do, scale: Optional[float] = None, causal: bool = False,
                   dq=None, dk=None, dv=None, workspace: Optional[torch.Tensor] = None,
                   opt: Optional[attn_options] = None, exp_mode: Optional[int] = None,
                   tau: Optional[float] = None, stream=None, variant: Optional[int] = None):
    """One phase of the backward (ATTN_BWD_*); the phases share ``workspace``."""
    B, Hq, Hkv, S, d = _dims(q, k)
    _need(q, "q", torch.bfloat16, (B, Hq, S, d))
    _need(k, "k", torch.bfloat16, (B, Hkv, S, d))
    _need(v, "v", torch.bfloat16, (B, Hkv, S, d))
    _need(o, "o", torch.bfloat16, (B, Hq, S, d))
    _need(lse, "lse", torch.float32, (B, Hq, S))
    _need(do, "do", torch.bfloat16, (B, Hq, S, d))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", torch.bfloat16, (B, Hq, S, d))
    _need(dk, "dk", torch.bfloat16, (B, Hkv, S, d))
    _need(dv, "dv", torch.bfloat16, (B, Hkv, S, d))
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor")
    _same_gpu(q=q, k=k, v=v, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv,
              **({} if workspace is None else {"workspace": workspace}))
    nbytes = attn_bwd_workspace_bytes(B, Hq, Hkv, S, d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    op = _options(opt, exp_mode, tau, variant)
    with _on(q.device):
        st = lib().attn_bwd_phase(int(phase), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                               _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, S, d, scale,
                               int(bool(causal)), _ptr(workspace),
                               workspace.numel() * workspace.element_size(),
                               None if op is None else ctypes.byref(op), _stream(stream))
    _check(st)
    return dq, dk, dv


def attn_bwd(q, k, v, o, lse, do, scale: Optional[float] = None, causal: bool = False,
             dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward pass with the default options (see attn_bwd_ex)."""
    return attn_bwd_ex(q, k, v, o, lse, do, scale, causal, dq, dk, dv, workspace, stream=stream)


ATTN_ERR_SCRATCH = 8


def attn_bwd_noalloc(q, k, v, o, lse, do, scale: Optional[float] = None, causal: bool = False,
                     dq=None, dk=None, dv=None, stream=None):
    """attn_bwd whose scratch is the library's static per-device buffer (64 MiB): no
    workspace argument and no allocation in the library.  Returns (dq, dk, dv); outputs
    not given are allocated here with torch.  Raises AttnError(ATTN_ERR_SCRATCH) for
    problems whose workspace exceeds the buffer.  Calls that overlap in time on one GPU
    race on the shared buffer."""
    B, Hq, Hkv, S, d = _dims(q, k)
    _need(q, "q", torch.bfloat16, (B, Hq, S, d))
    _need(k, "k", torch.bfloat16, (B, Hkv, S, d))
    _need(v, "v", torch.bfloat16, (B, Hkv, S, d))
    _need(o, "o", torch.bfloat16, (B, Hq, S, d))
    _need(lse, "lse", torch.float32, (B, Hq, S))
    _need(do, "do", torch.bfloat16, (B, Hq, S, d))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", torch.bfloat16, (B, Hq, S, d))
    _need(dk, "dk", torch.bfloat16, (B, Hkv, S, d))
    _need(dv, "dv", torch.bfloat16, (B, Hkv, S, d))
    _same_gpu(q=q, k=k, v=v, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with _on(q.device):
        st = lib().attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                    _ptr(dv), B, Hq, Hkv, S, d, scale, int(bool(causal)), _stream(stream))
    _check(st)
    return dq, dk, dv


def attn_exp2_eval(x: torch.Tensor, exp_mode: int = ATTN_EXP_HW, stream=None) -> torch.Tensor:
    """2^x on the GPU with the kernels' exp2 (x: fp32 GPU tensor)."""
    if x.device.type != "cuda" or x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp32 GPU tensor")
    y = torch.empty_like(x)
    with torch.cuda.device(x.device):
        _check(lib().attn_exp2_eval(_ptr(x), _ptr(y), x.numel(), int(exp_mode), _stream(stream)))
    return y


def attn_exp2_poly_host(x) -> "numpy.ndarray":  # noqa: F821
    """Host evaluation of the cubic-polynomial exp2 (numpy float32 in, float32 out)."""
    import numpy as np
    xa = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    y = np.empty_like(xa)
    lib().attn_exp2_poly_host(xa.ctypes.data_as(ctypes.c_void_p), y.ctypes.data_as(ctypes.c_void_p), xa.size)
    return y


class _Attention(torch.autograd.Function):
    """attn_fwd in the forward, attn_bwd in the backward (O and LSE kept for it)."""

    @staticmethod
    def forward(ctx, q, k, v, scale, causal):
        o, lse = attn_fwd(q, k, v, scale, causal)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale, ctx.causal = scale, causal
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = attn_bwd(q, k, v, o, lse, do.contiguous(), ctx.scale, ctx.causal)
        return dq, dk, dv, None, None


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
              causal: bool = False, return_lse: bool = False):
    """Exact attention with autograd: O = softmax(scale Q K^T [causal mask]) V on bf16
    [B, Hq, S, d] Q and [B, Hkv, S, d] K, V (contiguous, one GPU), computed by attn_fwd;
    the gradients of Q, K and V come from attn_bwd (so the incoming gradient of O is taken
    as bf16, contiguous).  Returns O, or (O, LSE) with return_lse (LSE [B, Hq, S] fp32,
    natural log, not differentiable)."""
    o, lse = _Attention.apply(q, k, v, scale, causal)
    return (o, lse) if return_lse else o


class _AttentionVarlen(torch.autograd.Function):
    """attn_fwd_varlen in the forward, attn_bwd_varlen in the backward (O and LSE kept)."""

    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens, max_seqlen, scale, causal):
        o, lse = attn_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, scale, causal)
        ctx.save_for_backward(q, k, v, o, lse, cu_seqlens)
        ctx.max_seqlen, ctx.scale, ctx.causal = max_seqlen, scale, causal
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        q, k, v, o, lse, cu = ctx.saved_tensors
        # Rows outside every sequence get no gradient from the library: zero them first.
        dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
        attn_bwd_varlen(q, k, v, o, lse, do.contiguous(), cu, ctx.max_seqlen, ctx.scale, ctx.causal,
                        dq=dq, dk=dk, dv=dv)
        return dq, dk, dv, None, None, None, None


def attention_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                     max_seqlen: int, scale: Optional[float] = None, causal: bool = False,
                     return_lse: bool = False):
    """Exact attention with autograd over a packed batch: attn_fwd_varlen's layouts
    (q [total, Hq, d], k and v [total, Hkv, d] bf16, cu_seqlens [nseq + 1] int32 on the
    same GPU, max_seqlen >= every length); gradients from attn_bwd_varlen (zero for rows
    outside every sequence).  Returns O, or (O, LSE [Hq, total]) with return_lse."""
    o, lse = _AttentionVarlen.apply(q, k, v, cu_seqlens, int(max_seqlen), scale, causal)
    return (o, lse) if return_lse else o
