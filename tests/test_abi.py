"""The C ABI without a GPU: the library loads, exports every declared symbol, and
rejects invalid arguments with the documented status before launching anything."""

import ctypes
import os
import re

import pytest

import exact_attention_27_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, HIP, VALUE = range(8)
A = ctypes.c_void_p(0x10000)  # aligned fake device pointers: never dereferenced on error paths
A2 = ctypes.c_void_p(0x20000)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ea.lib()
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"libattn.so does not export {n}"


def test_python_binding_has_the_c_names():
    for n in declared_functions():
        assert hasattr(ea, n), f"binding lacks {n}"


def test_default_options():
    o = ea.attn_default_options()
    assert o.exp_mode in (ea.ATTN_EXP_HW, ea.ATTN_EXP_POLY3)
    assert 0.0 <= o.tau <= 30.0 and o.variant == ea.ATTN_VARIANT_AUTO


def test_status_strings():
    for s in range(9):
        assert ea.attn_status_string(s).startswith("ATTN_")
    assert "unknown" in ea.attn_status_string(99)


def fwd(q=A, k=A, v=A, o=A, lse=A, B=1, Hq=2, Hkv=1, S=8, d=64, scale=0.125, causal=0, opt=None):
    lib = ea.lib()
    if opt is None:
        return lib.attn_fwd(q, k, v, o, lse, B, Hq, Hkv, S, d, scale, causal, None)
    return lib.attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, S, d, scale, causal, ctypes.byref(opt), None)


def bwd(ptrs=None, B=1, Hq=2, Hkv=1, S=8, d=64, scale=0.125, causal=0, ws=A2, wsb=None, opt=None):
    lib = ea.lib()
    p = [A] * 9 if ptrs is None else ptrs
    if wsb is None:
        wsb = ea.attn_bwd_workspace_bytes(B, Hq, Hkv, S, d)
    args = p + [B, Hq, Hkv, S, d, scale, causal, ws, wsb]
    if opt is None:
        return lib.attn_bwd(*args, None)
    return lib.attn_bwd_ex(*args, ctypes.byref(opt), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(o=None), NULL), (dict(lse=None), NULL),
    (dict(Hq=3, Hkv=2), SHAPE), (dict(Hkv=0), SHAPE), (dict(Hq=0), SHAPE), (dict(S=-1), SHAPE), (dict(B=-2), SHAPE),
    (dict(d=96), UNSUP), (dict(d=256), UNSUP), (dict(d=0), UNSUP),
    (dict(q=ctypes.c_void_p(0x10008)), ALIGN), (dict(lse=ctypes.c_void_p(0x10004)), ALIGN),
    (dict(scale=float("nan")), VALUE), (dict(scale=float("inf")), VALUE),
    (dict(S=1 << 30, B=1 << 10, Hq=64, Hkv=64), SHAPE),
])
def test_fwd_rejects(kw, status):
    assert fwd(**kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(S=0), dict(B=0, q=None, k=None, v=None, o=None, lse=None)])
def test_fwd_empty_is_ok_without_launch(kw):
    assert fwd(**kw) == OK


@pytest.mark.parametrize("opt,status", [
    (ea.attn_options(5, 8.0, 0), UNSUP), (ea.attn_options(0, 8.0, 3), UNSUP), (ea.attn_options(0, 8.0, 4), UNSUP), (ea.attn_options(0, 8.0, -1), UNSUP),
    (ea.attn_options(0, -1.0, 0), VALUE), (ea.attn_options(0, float("nan"), 0), VALUE), (ea.attn_options(1, 31.0, 0), VALUE),
])
def test_fwd_rejects_options(opt, status):
    assert fwd(opt=opt) == status


def test_grid_limits():
    """Sizes whose launch grids would not fit in 31 bits are rejected before any launch
    (the first passes every other limit but the backward preprocess grid, 64 workgroups
    per (batch, KV head))."""
    assert ea.attn_bwd_workspace_bytes(1 << 25, 1, 1, 1, 64) == 0
    assert fwd(B=1 << 25, Hq=1, Hkv=1, S=1, d=64) == SHAPE
    assert ea.attn_bwd_workspace_bytes((1 << 25) - 1, 1, 1, 1, 64) > 0
    assert fwd(B=1, Hq=1, Hkv=1, S=1 << 24, d=128) == SHAPE  # row offsets within a head
    assert fwd(B=1 << 20, Hq=1 << 10, Hkv=1, S=1 << 8, d=64) == SHAPE


def test_workspace_bytes():
    B, Hq, Hkv, S, d = 2, 4, 2, 100, 128
    rup = lambda x: (x + 255) // 256 * 256
    prows = B * Hq * ((S + 63) // 64 * 64)
    rows = 3 * rup(prows * 4)                    # -D from O, LSE log2 e, -D defined
    maxima = rup(B * Hkv * 64 * 4 * 4)           # partial maxima of |dO|, |V|, |Q|, |K|
    f16 = 2 * rup(B * Hq * S * d * 2)            # dO and Q in fp16
    assert ea.attn_bwd_workspace_bytes(B, Hq, Hkv, S, d) == rows + maxima + f16
    assert ea.attn_bwd_workspace_bytes(0, Hq, Hkv, S, d) == 0
    assert ea.attn_bwd_workspace_bytes(B, 3, 2, S, d) == 0
    assert ea.attn_bwd_workspace_bytes(B, Hq, Hkv, S, 80) == 0


@pytest.mark.parametrize("i", range(9))
def test_bwd_rejects_null(i):
    p = [A] * 9
    p[i] = None
    assert bwd(ptrs=p) == NULL


@pytest.mark.parametrize("i", range(9))
def test_bwd_rejects_misaligned(i):
    p = [A] * 9
    p[i] = ctypes.c_void_p(0x10002)
    assert bwd(ptrs=p) == ALIGN


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), WS), (dict(wsb=16), WS), (dict(ws=ctypes.c_void_p(0x20010)), WS),
    (dict(Hq=4, Hkv=3), SHAPE), (dict(d=32), UNSUP), (dict(scale=float("-inf")), VALUE),
    (dict(opt=ea.attn_options(0, 100.0, 0)), VALUE), (dict(B=0, ws=None), OK), (dict(S=0), OK),
])
def test_bwd_rejects(kw, status):
    assert bwd(**kw) == status


def test_exp2_eval_rejects():
    lib = ea.lib()
    assert lib.attn_exp2_eval(A, A, -1, 0, None) == SHAPE
    assert lib.attn_exp2_eval(A, A, 4, 7, None) == UNSUP
    assert lib.attn_exp2_eval(None, A, 4, 0, None) == NULL
    assert lib.attn_exp2_eval(None, None, 0, 0, None) == OK


def test_bwd_phase_rejects_unknown_phase():
    lib = ea.lib()
    args = [A] * 9 + [1, 2, 1, 8, 64, 0.125, 0, A2, ea.attn_bwd_workspace_bytes(1, 2, 1, 8, 64)]
    assert lib.attn_bwd_phase(7, *args, None, None) == UNSUP
    assert lib.attn_bwd_phase(-1, *args, None, None) == UNSUP
    p = list(args)
    p[0] = None
    assert lib.attn_bwd_phase(2, *p, None, None) == NULL


def fwd_varlen(q=A, k=A, v=A, o=A, lse=A, cu=ctypes.c_void_p(0x30000), nseq=2, total=16, max_seqlen=8, Hq=2, Hkv=1,
               d=64, scale=0.125, causal=0, opt=None):
    lib = ea.lib()
    return lib.attn_fwd_varlen(q, k, v, o, lse, cu, nseq, total, max_seqlen, Hq, Hkv, d, scale, causal,
                               None if opt is None else ctypes.byref(opt), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(o=None), NULL), (dict(lse=None), NULL),
    (dict(cu=None), NULL),
    (dict(nseq=-1), SHAPE), (dict(total=-1), SHAPE), (dict(max_seqlen=-1), SHAPE), (dict(Hq=3, Hkv=2), SHAPE),
    (dict(Hkv=0), SHAPE), (dict(nseq=1 << 30, max_seqlen=1 << 30, Hq=64, Hkv=64), SHAPE),
    (dict(d=96), UNSUP), (dict(opt=ea.attn_options(4, 8.0, 0)), UNSUP),
    (dict(v=ctypes.c_void_p(0x10008)), ALIGN), (dict(cu=ctypes.c_void_p(0x30002)), ALIGN),
    (dict(scale=float("nan")), VALUE), (dict(opt=ea.attn_options(0, -2.0, 0)), VALUE),
])
def test_fwd_varlen_rejects(kw, status):
    assert fwd_varlen(**kw) == status


@pytest.mark.parametrize("kw", [dict(nseq=0), dict(total=0), dict(max_seqlen=0),
                                dict(nseq=0, q=None, k=None, v=None, o=None, lse=None, cu=None)])
def test_fwd_varlen_empty_is_ok_without_launch(kw):
    assert fwd_varlen(**kw) == OK


def test_fwd_varlen_binding_checks_arguments():
    """Operand checks run before the device check, so CPU tensors reach each of them."""
    import torch
    q = torch.zeros(10, 2, 64, dtype=torch.bfloat16)
    k = torch.zeros(10, 1, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 10], dtype=torch.int32)
    with pytest.raises(ValueError, match="cu_seqlens must be"):
        ea.attn_fwd_varlen(q, k, k, torch.tensor([0, 10], dtype=torch.int64), 10)
    with pytest.raises(ValueError, match="has shape"):
        ea.attn_fwd_varlen(q, k, k[:9], cu, 10)
    with pytest.raises(TypeError, match="must be torch.bfloat16"):
        ea.attn_fwd_varlen(q, k, k.float(), cu, 10)
    with pytest.raises(ValueError, match="must be on a GPU device"):
        ea.attn_fwd_varlen(q, k, k, cu, 10)


def test_fwd_binding_checks_arguments():
    import torch
    q = torch.zeros(1, 4, 32, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 32, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q must be"):
        ea.attn_fwd(q[0], k, k)
    with pytest.raises(ValueError, match="has shape"):
        ea.attn_fwd(q, k, k[:, :, :16])
    with pytest.raises(TypeError, match="must be torch.bfloat16"):
        ea.attn_fwd(q, k.half(), k)
    with pytest.raises(ValueError, match="contiguous"):
        ea.attn_fwd(q, k.transpose(2, 3).contiguous().transpose(2, 3), k)
    with pytest.raises(ValueError, match="has shape"):
        ea.attn_fwd(q, k, k, o=torch.zeros(1, 4, 32, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="must be on a GPU device"):
        ea.attn_fwd(q, k, k)


def test_bwd_binding_checks_arguments():
    import torch
    q = torch.zeros(1, 4, 32, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 32, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 4, 32)
    with pytest.raises(ValueError, match="has shape"):
        ea.attn_bwd(q, k, k, q, lse[:, :, :16], q)
    with pytest.raises(TypeError, match="must be torch.float32"):
        ea.attn_bwd(q, k, k, q, lse.double(), q)
    with pytest.raises(ValueError, match="workspace must be"):
        ea.attn_bwd(q, k, k, q, lse, q, workspace=torch.zeros(64, dtype=torch.uint8)[::2])
    with pytest.raises(ValueError, match="must be on a GPU device"):
        ea.attn_bwd(q, k, k, q, lse, q)


def test_noalloc_checks_before_any_hip_call():
    """attn_bwd_noalloc validates like attn_bwd and rejects problems whose workspace
    exceeds its static 64 MiB scratch, all before any HIP call (no GPU here)."""
    lib = ea.lib()
    SCRATCH = 8
    assert ea.ATTN_ERR_SCRATCH == SCRATCH

    def call(ptrs=None, B=1, Hq=2, Hkv=1, S=8, d=64, scale=0.125):
        p = [A] * 9 if ptrs is None else ptrs
        return lib.attn_bwd_noalloc(*p, B, Hq, Hkv, S, d, scale, 1, None)

    assert call(B=0) == OK
    assert call(Hq=3, Hkv=2) == SHAPE
    assert call(d=80) == UNSUP
    assert call(scale=float("inf")) == VALUE
    assert call(ptrs=[A] * 8 + [None]) == NULL
    assert call(ptrs=[A] * 8 + [ctypes.c_void_p(0x10008)]) == ALIGN
    assert ea.attn_bwd_workspace_bytes(1, 16, 16, 8192, 128) > 64 << 20
    assert call(B=1, Hq=16, Hkv=16, S=8192, d=128) == SCRATCH
    assert "64 MiB" in ea.attn_status_string(SCRATCH)


def bwd_varlen(q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A, cu=ctypes.c_void_p(0x30000), nseq=2, total=16,
               max_seqlen=8, Hq=2, Hkv=1, d=64, scale=0.125, causal=0, ws=A2, wsb=None, opt=None):
    lib = ea.lib()
    if wsb is None:
        wsb = max(ea.attn_bwd_varlen_workspace_bytes(nseq, total, Hq, Hkv, d), 1)
    return lib.attn_bwd_varlen(q, k, v, o, lse, do, dq, dk, dv, cu, nseq, total, max_seqlen, Hq, Hkv, d, scale,
                               causal, ws, wsb, None if opt is None else ctypes.byref(opt), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(o=None), NULL), (dict(lse=None), NULL),
    (dict(do=None), NULL), (dict(dq=None), NULL), (dict(dk=None), NULL), (dict(dv=None), NULL), (dict(cu=None), NULL),
    (dict(nseq=-1), SHAPE), (dict(total=-1), SHAPE), (dict(max_seqlen=-1), SHAPE), (dict(Hq=3, Hkv=2), SHAPE),
    (dict(Hkv=0), SHAPE), (dict(nseq=1 << 30, max_seqlen=1 << 30, Hq=64, Hkv=64), SHAPE),
    (dict(d=96), UNSUP), (dict(opt=ea.attn_options(4, 8.0, 0)), UNSUP),
    (dict(dk=ctypes.c_void_p(0x10008)), ALIGN), (dict(cu=ctypes.c_void_p(0x30002)), ALIGN),
    (dict(scale=float("inf")), VALUE),
    (dict(ws=None), WS), (dict(wsb=64), WS), (dict(ws=ctypes.c_void_p(0x20010)), WS),
])
def test_bwd_varlen_rejects(kw, status):
    assert bwd_varlen(**kw) == status


@pytest.mark.parametrize("kw", [dict(nseq=0), dict(total=0), dict(max_seqlen=0),
                                dict(total=0, q=None, dq=None, cu=None, ws=None)])
def test_bwd_varlen_empty_is_ok_without_launch(kw):
    assert bwd_varlen(**kw) == OK


def test_bwd_varlen_binding_checks_arguments():
    """Operand checks run before the device check, so CPU tensors reach each of them."""
    import torch
    q = torch.zeros(10, 2, 64, dtype=torch.bfloat16)
    k = torch.zeros(10, 1, 64, dtype=torch.bfloat16)
    lse = torch.zeros(2, 10, dtype=torch.float32)
    cu = torch.tensor([0, 10], dtype=torch.int32)
    with pytest.raises(ValueError, match="cu_seqlens must be"):
        ea.attn_bwd_varlen(q, k, k, q, lse, q, torch.tensor([0, 10], dtype=torch.int64), 10)
    with pytest.raises(ValueError, match="has shape"):
        ea.attn_bwd_varlen(q, k, k, q, lse[:, :9], q, cu, 10)
    with pytest.raises(TypeError, match="must be torch.bfloat16"):
        ea.attn_bwd_varlen(q, k, k, q, lse, q.float(), cu, 10)
    with pytest.raises(ValueError, match="must be on a GPU device"):
        ea.attn_bwd_varlen(q, k, k, q, lse, q, cu, 10)


def test_varlen_workspace_bytes():
    """The packed backward's workspace grows with the tokens: per query head 64 (nseq +
    ceil(total / 64)) rows of the three fp32 row arrays and the two fp16 copies, plus the
    preprocess's partial maxima per (sequence, KV head)."""
    nseq, total, Hq, Hkv, d = 3, 1000, 4, 2, 128
    rup = lambda x: (x + 255) // 256 * 256
    prows = Hq * 64 * (nseq + (total + 63) // 64)
    want = 3 * rup(prows * 4) + rup(nseq * Hkv * 64 * 4 * 4) + 2 * rup(prows * d * 2)
    assert ea.attn_bwd_varlen_workspace_bytes(nseq, total, Hq, Hkv, d) == want
    # 1000 sequences of mean 500 with one of 32k: tokens, not nseq x the longest
    assert ea.attn_bwd_varlen_workspace_bytes(1000, 500_000, 32, 8, 128) < 10e9
    assert ea.attn_bwd_varlen_workspace_bytes(0, total, Hq, Hkv, d) == 0
    assert ea.attn_bwd_varlen_workspace_bytes(nseq, 0, Hq, Hkv, d) == 0
    assert ea.attn_bwd_varlen_workspace_bytes(nseq, total, 3, 2, d) == 0
    assert ea.attn_bwd_varlen_workspace_bytes(nseq, total, Hq, Hkv, 80) == 0
