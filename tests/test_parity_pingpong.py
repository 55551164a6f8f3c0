"""GPU parity of both forward schedules against the fp64 oracle: the ping-pong schedule
(attn_options.variant = 1: 8-wave workgroups whose two halves run half a step apart,
64-key tiles) and the four-wave schedule (variant 2: 32-key tiles, three waves per
SIMD), on edge shapes, options, every forward workload at full size (sampled rows of
every head) and packed (variable-length) batches.  The schedules round differently
(different tiles move the rescale points and the row-sum order), so each is compared
with the oracle; the automatic choice (variant 0, the default) equals, bit for bit, the
schedule it picks, and each schedule is deterministic.
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
def test_schedules_edge_shapes(case, causal):
    B, Hq, Hkv, S, d = case
    t = {n: x.to(DEV) for n, x in workloads.make_tensors(B, Hq, Hkv, S, d, seed=sum(case) + 7).items()}
    scale = d ** -0.5
    ro, rl = oracle.attention_forward(f64(t["q"]), f64(t["k"]), f64(t["v"]), scale, causal)
    for variant in (PP, FW):
        print(f"\n[schedule {variant} fwd] {case} causal={causal}", flush=True)
        o, lse = ea.attn_fwd_ex(t["q"], t["k"], t["v"], scale, causal, variant=variant)
        o2, l2 = ea.attn_fwd_ex(t["q"], t["k"], t["v"], scale, causal, variant=variant)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, l2)  # deterministic
        assert_bf16_close("o", o, ro)
        assert_lse_close(lse, rl)


@pytest.mark.parametrize("exp_mode", [ea.ATTN_EXP_HW, ea.ATTN_EXP_POLY3])
@pytest.mark.parametrize("tau", [0.0, 30.0])
def test_schedules_options(exp_mode, tau):
    B, Hq, Hkv, S, d = 1, 4, 2, 700, 128
    t = {n: x.to(DEV) for n, x in workloads.make_tensors(B, Hq, Hkv, S, d, seed=77).items()}
    ro, rl = oracle.attention_forward(f64(t["q"]), f64(t["k"]), f64(t["v"]), d ** -0.5, True)
    for variant in (PP, FW):
        print(f"\n[schedule {variant} options] exp_mode={exp_mode} tau={tau}", flush=True)
        o, lse = ea.attn_fwd_ex(t["q"], t["k"], t["v"], d ** -0.5, True, exp_mode=exp_mode, tau=tau, variant=variant)
        torch.cuda.synchronize()
        assert_bf16_close("o", o, ro)
        assert_lse_close(lse, rl)


def _auto_schedule(w):
    """The schedule ATTN_VARIANT_AUTO picks for a dense launch (as the library documents)."""
    pp = (not w.causal) and w.S >= 8192 and w.B * w.Hq * ((w.S + 255) // 256) >= 256
    return PP if pp else FW


def _sample_rows(S, seed, n=24):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, S - 1, S // 2], g.choice(S, size=min(n, S), replace=False)]))


@pytest.mark.parametrize("wn", [1, 2, 3, 5, 6, 7, 8])
def test_schedules_on_workloads(wn):
    """Each schedule on the full-size forward workloads, against the oracle on sampled
    rows of every head; the default equals the schedule it picks."""
    w = workloads.WORKLOADS[wn]
    host = workloads.make_inputs(w)
    t = {n: x.to(DEV) for n, x in host.items() if n in ("q", "k", "v")}
    outs = {}
    for variant in (PP, FW, ea.ATTN_VARIANT_AUTO):
        outs[variant] = ea.attn_fwd_ex(t["q"], t["k"], t["v"], w.scale, w.causal, variant=variant)
    torch.cuda.synchronize()
    auto = _auto_schedule(w)
    print(f"\n[schedules] {w.name}: {w.describe()}; default picks {auto}", flush=True)
    assert torch.equal(outs[ea.ATTN_VARIANT_AUTO][0], outs[auto][0])
    assert torch.equal(outs[ea.ATTN_VARIANT_AUTO][1], outs[auto][1])
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    refs = {}
    for b, h in heads:
        rows = _sample_rows(w.S, 100 * wn + b * w.Hq + h)
        hk = h // w.group
        refs[(b, h)] = (rows, oracle.head_forward(f64(host["q"][b, h]), f64(host["k"][b, hk]), f64(host["v"][b, hk]),
                                                  w.scale, w.causal, rows=rows))
    for variant in (PP, FW):
        o, lse = outs[variant][0].cpu(), outs[variant][1].cpu()
        go = torch.cat([o[b, h][torch.from_numpy(refs[(b, h)][0])] for b, h in heads])
        gl = torch.cat([lse[b, h][torch.from_numpy(refs[(b, h)][0])] for b, h in heads])
        print(f"schedule {variant}:", flush=True)
        assert_bf16_close("o", go, np.concatenate([refs[k][1][0] for k in heads]))
        assert_lse_close(gl, np.concatenate([refs[k][1][1] for k in heads]))


@pytest.mark.parametrize("causal", [False, True])
def test_pingpong_varlen(causal):
    """Ragged packed batch: each schedule against the oracle on sampled rows of every
    sequence; the default equals the four-wave schedule; rows past max_seqlen left alone."""
    lengths = [700, 0, 1, 255, 257, 64, 1300]
    Hq, Hkv, d = 4, 2, 128
    print(f"\n[pingpong varlen] lengths={lengths} causal={causal}", flush=True)
    t = workloads.make_varlen_tensors(lengths, Hq, Hkv, d, seed=31)
    dev = {n: x.to(DEV) for n, x in t.items()}
    total = int(t["q"].shape[0])
    outs = {}
    for variant in (PP, FW, ea.ATTN_VARIANT_AUTO):
        o = torch.full((total, Hq, d), 12288.0, dtype=torch.bfloat16, device=DEV)
        lse = torch.full((Hq, total), 12288.0, dtype=torch.float32, device=DEV)
        ea.attn_fwd_varlen(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], 1000, d ** -0.5, causal, o=o, lse=lse,
                           variant=variant)
        outs[variant] = (o, lse)
    torch.cuda.synchronize()
    # packed batches always take the four-wave schedule by default
    assert torch.equal(outs[ea.ATTN_VARIANT_AUTO][0], outs[FW][0])
    assert torch.equal(outs[ea.ATTN_VARIANT_AUTO][1], outs[FW][1])
    cu = t["cu_seqlens"].tolist()
    for variant in (PP, FW):
        o, lse = outs[variant][0].cpu(), outs[variant][1].cpu()
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
        print(f"schedule {variant}:", flush=True)
        assert_bf16_close("o", torch.cat(go), np.concatenate(ro))
        assert_lse_close(torch.cat(gl), np.concatenate(rl))
