"""GPU parity on small and edge shapes: the HIP kernels against the fp64 oracle.

Shapes span several tiles and ragged tails (S not a multiple of the 64-key and
128-query tiles), both head sizes, causal and not, GQA groups 1-8, both exp2
evaluations, and rescale thresholds 0 (rescale on every growth) and 8.
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


def inputs(B, Hq, Hkv, S, d, seed):
    t = workloads.make_tensors(B, Hq, Hkv, S, d, seed)
    return {n: x.to(DEV) for n, x in t.items()}


def oracle_fwd(t, scale, causal):
    return oracle.attention_forward(f64(t["q"]), f64(t["k"]), f64(t["v"]), scale, causal)


FWD_CASES = [
    # (B, Hq, Hkv, S, d)
    (1, 1, 1, 1, 64), (1, 2, 1, 17, 64), (2, 2, 2, 64, 128), (1, 1, 1, 127, 128), (1, 2, 2, 128, 64),
    (1, 4, 2, 129, 128), (2, 4, 1, 257, 64), (1, 8, 1, 200, 128), (1, 8, 2, 384, 128), (1, 2, 2, 1000, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "B%dHq%dHkv%dS%dd%d" % c)
def test_fwd_edge_shapes(case, causal):
    B, Hq, Hkv, S, d = case
    print(f"\n[fwd] {case} causal={causal}", flush=True)
    t = inputs(B, Hq, Hkv, S, d, seed=sum(case))
    scale = d ** -0.5
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], scale, causal)
    torch.cuda.synchronize()
    ro, rlse = oracle_fwd(t, scale, causal)
    assert_bf16_close("o", o, ro)
    assert_lse_close(lse, rlse)
    if causal:  # query 0 sees key 0 only: O_0 is V_0 bit for bit
        G = Hq // Hkv
        for h in range(Hq):
            assert torch.equal(o[:, h, 0], t["v"][:, h // G, 0])


@pytest.mark.parametrize("exp_mode", [ea.ATTN_EXP_HW, ea.ATTN_EXP_POLY3])
@pytest.mark.parametrize("tau", [0.0, 8.0, 30.0])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_options(exp_mode, tau, causal):
    B, Hq, Hkv, S, d = 1, 4, 2, 333, 128
    print(f"\n[fwd opt] exp_mode={exp_mode} tau={tau} causal={causal}", flush=True)
    t = inputs(B, Hq, Hkv, S, d, seed=7)
    o, lse = ea.attn_fwd_ex(t["q"], t["k"], t["v"], d ** -0.5, causal, exp_mode=exp_mode, tau=tau)
    torch.cuda.synchronize()
    ro, rlse = oracle_fwd(t, d ** -0.5, causal)
    assert_bf16_close("o", o, ro)
    assert_lse_close(lse, rlse)


@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_fwd_rescale_with_growing_scores(tau):
    """Scores that grow along the keys force the running maximum up on every tile:
    K rows scaled by a ramp, plus a large shift of K along Q's mean direction."""
    B, Hq, Hkv, S, d = 1, 2, 2, 520, 64
    print(f"\n[fwd growing] tau={tau}", flush=True)
    t = inputs(B, Hq, Hkv, S, d, seed=11)
    ramp = torch.linspace(0.2, 4.0, S, device=DEV).view(1, 1, S, 1)
    t["k"] = (t["k"].float() * ramp + 0.5).to(torch.bfloat16)
    o, lse = ea.attn_fwd_ex(t["q"], t["k"], t["v"], d ** -0.5, True, tau=tau)
    torch.cuda.synchronize()
    ro, rlse = oracle_fwd(t, d ** -0.5, True)
    assert_bf16_close("o", o, ro)
    assert_lse_close(lse, rlse)


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.5, 3.0])
def test_fwd_scales(scale):
    """Negative, zero and large scales (any finite scale is accepted)."""
    B, Hq, Hkv, S, d = 1, 2, 1, 150, 64
    print(f"\n[fwd scale] {scale}", flush=True)
    t = inputs(B, Hq, Hkv, S, d, seed=13)
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], scale, True)
    torch.cuda.synchronize()
    ro, rlse = oracle_fwd(t, scale, True)
    assert_bf16_close("o", o, ro)
    assert_lse_close(lse, rlse, max_abs=1e-3 * max(1.0, abs(scale) * 4))


def test_fwd_deterministic_and_stream():
    """The forward is deterministic and runs on a caller-provided stream."""
    t = inputs(2, 4, 2, 300, 128, seed=17)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o1, l1 = ea.attn_fwd(t["q"], t["k"], t["v"], None, True, stream=s)
        o2, l2 = ea.attn_fwd(t["q"], t["k"], t["v"], None, True, stream=s)
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_empty():
    q = torch.empty((0, 2, 16, 64), dtype=torch.bfloat16, device=DEV)
    o, lse = ea.attn_fwd(q, q[:, :1], q[:, :1])
    assert o.numel() == 0 and lse.numel() == 0
    q = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device=DEV)
    o, lse = ea.attn_fwd(q, q, q)
    assert o.numel() == 0
