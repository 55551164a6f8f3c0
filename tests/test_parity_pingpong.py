"""GPU parity of the ping-pong forward schedule (attn_options.variant = 1: 8-wave
workgroups whose two halves run half a step apart) against the fp64 oracle on edge
shapes, and bit for bit against the four-wave schedule (variant 2) on every forward
workload at full size and on packed (variable-length) batches; the automatic choice
(variant 0, the default) equals both.  The schedules perform the same arithmetic in the
same order for every output, so equality is exact.
"""

import numpy as np
import pytest
import torch

import exact_attention_27_amd as ea
import oracle
import workloads
from helpers import assert_bf16_close, assert_lse_close, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PP = ea.ATTN_VARIANT_PINGPONG
FW = ea.ATTN_VARIANT_FOURWAVE

EDGE = [
    # (B, Hq, Hkv, S, d): one tile, ragged tails on both sides of the 256-query workgroup
    (1, 1, 1, 1, 64), (1, 2, 1, 63, 128), (1, 4, 2, 255, 128), (1, 2, 2, 257, 64), (2, 8, 2, 513, 128),
    (1, 4, 4, 1000, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", EDGE, ids=lambda c: "B%dHq%dHkv%dS%dd%d" % c)
def test_pingpong_edge_shapes(case, causal):
    B, Hq, Hkv, S, d = case
    print(f"\n[pingpong fwd] {case} causal={causal}", flush=True)
    t = {n: x.to(DEV) for n, x in workloads.make_tensors(B, Hq, Hkv, S, d, seed=sum(case) + 7).items()}
    scale = d ** -0.5
    o, lse = ea.attn_fwd_ex(t["q"], t["k"], t["v"], scale, causal, variant=PP)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward(f64(t["q"]), f64(t["k"]), f64(t["v"]), scale, causal)
    assert_bf16_close("o", o, ro)
    assert_lse_close(lse, rl)
    o0, l0 = ea.attn_fwd_ex(t["q"], t["k"], t["v"], scale, causal, variant=FW)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, l0)


@pytest.mark.parametrize("exp_mode", [ea.ATTN_EXP_HW, ea.ATTN_EXP_POLY3])
@pytest.mark.parametrize("tau", [0.0, 30.0])
def test_pingpong_options(exp_mode, tau):
    B, Hq, Hkv, S, d = 1, 4, 2, 700, 128
    print(f"\n[pingpong options] exp_mode={exp_mode} tau={tau}", flush=True)
    t = {n: x.to(DEV) for n, x in workloads.make_tensors(B, Hq, Hkv, S, d, seed=77).items()}
    o, lse = ea.attn_fwd_ex(t["q"], t["k"], t["v"], d ** -0.5, True, exp_mode=exp_mode, tau=tau, variant=PP)
    o0, l0 = ea.attn_fwd_ex(t["q"], t["k"], t["v"], d ** -0.5, True, exp_mode=exp_mode, tau=tau, variant=FW)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, l0)


@pytest.mark.parametrize("wn", [1, 2, 3, 5, 6, 7, 8])
def test_pingpong_equals_fourwave_on_workloads(wn):
    w = workloads.WORKLOADS[wn]
    print(f"\n[pingpong == fourwave == auto] {w.name}: {w.describe()}", flush=True)
    t = {n: x.to(DEV) for n, x in workloads.make_inputs(w).items() if n in ("q", "k", "v")}
    o, lse = ea.attn_fwd_ex(t["q"], t["k"], t["v"], w.scale, w.causal, variant=PP)
    o0, l0 = ea.attn_fwd_ex(t["q"], t["k"], t["v"], w.scale, w.causal, variant=FW)
    oa, la = ea.attn_fwd(t["q"], t["k"], t["v"], w.scale, w.causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, l0)
    assert torch.equal(oa, o0) and torch.equal(la, l0)


@pytest.mark.parametrize("causal", [False, True])
def test_pingpong_varlen(causal):
    """Ragged packed batch: equal to the default schedule; a sampled check against the
    oracle on every sequence; rows past max_seqlen left alone."""
    lengths = [700, 0, 1, 255, 257, 64, 1300]
    Hq, Hkv, d = 4, 2, 128
    print(f"\n[pingpong varlen] lengths={lengths} causal={causal}", flush=True)
    t = workloads.make_varlen_tensors(lengths, Hq, Hkv, d, seed=31)
    dev = {n: x.to(DEV) for n, x in t.items()}
    total = int(t["q"].shape[0])
    outs = []
    for variant in (PP, FW, ea.ATTN_VARIANT_AUTO):
        o = torch.full((total, Hq, d), 12288.0, dtype=torch.bfloat16, device=DEV)
        lse = torch.full((Hq, total), 12288.0, dtype=torch.float32, device=DEV)
        ea.attn_fwd_varlen(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], 1000, d ** -0.5, causal, o=o, lse=lse,
                           variant=variant)
        outs.append((o, lse))
    torch.cuda.synchronize()
    for other in outs[1:]:
        assert torch.equal(outs[0][0], other[0]) and torch.equal(outs[0][1], other[1])
    o, lse = outs[0][0].cpu(), outs[0][1].cpu()
    cu = t["cu_seqlens"].tolist()
    a = cu[6]
    assert (o[a + 1000:a + 1300].float() == 12288.0).all()  # past max_seqlen: not written
    go, gl, ro, rl = [], [], [], []
    for s, n in enumerate(lengths):
        if n == 0:
            continue
        a = cu[s]
        rows = np.unique(np.array([0, n // 3, n // 2, min(n, 1000) - 1]))
        for h in range(Hq):
            x, y = oracle.head_forward(f64(t["q"][a:a + n, h]), f64(t["k"][a:a + n, h // 2]),
                                       f64(t["v"][a:a + n, h // 2]), d ** -0.5, causal, rows=rows)
            go.append(o[a + rows, h]); gl.append(lse[h, a + rows]); ro.append(x); rl.append(y)
    assert_bf16_close("o", torch.cat(go), np.concatenate(ro))
    assert_lse_close(torch.cat(gl), np.concatenate(rl))
