"""GPU: launches large enough to run in dispatch chunks.

When the operands that the workgroups of one (batch, KV head) group re-read (K and V for
the forward and the dQ kernel, the fp16 Q and dO of the group's query heads for the
dK/dV kernel) exceed 160 MiB over all groups, and sequences have at most 4096 keys, the
kernels take their grid in chunks of groups, one after the other.  Only the order of the
workgroups changes, never their arithmetic, so a batch run whole must equal, bit for bit,
the same batch run in slices small enough to be one chunk each (the small-shape parity
tests cover single-chunk launches against the oracle).  One KV group in the first chunk
and one in the last are also checked against the fp64 oracle.
"""

import pytest
import torch

import exact_attention_27_amd as ea
import oracle
import workloads
from helpers import assert_bf16_close, assert_lse_close, f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CASES = [
    # (B, Hq, Hkv, S, d, slices): 355 groups of 512,000 bytes of K and V (173 MiB): the
    # forward, dQ and dK/dV kernels run chunks of 184 and 171 groups (the last not a
    # multiple of 8, so its heads take the plain order).
    (71, 5, 5, 1000, 128, (0, 36, 71)),
    # 96 groups of 4 query heads: the dK/dV kernel's fp16 Q and dO are 2,048,000 bytes per
    # group (188 MiB): two chunks of 48; the forward and dQ kernels run one chunk.
    (24, 16, 4, 1000, 128, (0, 12, 24)),
    # d = 64: 660 groups of 256,000 bytes (161 MiB): chunks of 336 and 324 groups in all
    # three kernels.
    (132, 5, 5, 1000, 64, (0, 66, 132)),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dHq%dHkv%dS%dd%d" % c[:5])
def test_chunked_launch_equals_slices(case, causal):
    B, Hq, Hkv, S, d, cuts = case
    G = Hq // Hkv
    ngrp = B * Hkv
    plan = ea.attn_launch_plan(B, Hq, Hkv, S, d, causal)
    assert plan["dkdv_chunk"] < ngrp  # the dK/dV kernel runs in chunks
    for lo, hi in zip(cuts[:-1], cuts[1:]):  # every slice is one chunk
        ps = ea.attn_launch_plan(hi - lo, Hq, Hkv, S, d, causal)
        n = (hi - lo) * Hkv
        assert ps["fwd_chunk"] == ps["dq_chunk"] == ps["dkdv_chunk"] == n
    print(f"\n[chunks] {case[:5]} causal={causal} plan {plan} of {ngrp} groups", flush=True)
    t = {n: x.to(DEV) for n, x in workloads.make_tensors(B, Hq, Hkv, S, d, seed=500 + B).items()}
    scale = d ** -0.5
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], scale, causal)
    dq, dk, dv = ea.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], scale, causal)
    torch.cuda.synchronize()
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        s = {n: x[lo:hi].contiguous() for n, x in t.items()}
        os_, lses = ea.attn_fwd(s["q"], s["k"], s["v"], scale, causal)
        gs = ea.attn_bwd(s["q"], s["k"], s["v"], os_, lses, s["do"], scale, causal)
        torch.cuda.synchronize()
        assert torch.equal(o[lo:hi], os_) and torch.equal(lse[lo:hi], lses), (lo, hi)
        for name, full, part in zip(("dq", "dk", "dv"), (dq, dk, dv), gs):
            assert torch.equal(full[lo:hi], part), (name, lo, hi)
        del s, os_, lses, gs
    # One KV group of the first chunk and the last group of the last chunk, against the oracle.
    for b, hkv in ((0, 0), (B - 1, Hkv - 1)):
        hs = slice(hkv * G, (hkv + 1) * G)
        q, k, v, do = (f64(t[n][b:b + 1, hs if n in ("q", "do") else slice(hkv, hkv + 1)]) for n in ("q", "k", "v", "do"))
        ro, rlse = oracle.attention_forward(q, k, v, scale, causal)
        rdq, rdk, rdv = oracle.attention_backward(q, k, v, do, scale, causal)
        assert_bf16_close("o", o[b:b + 1, hs], ro)
        assert_lse_close(lse[b:b + 1, hs], rlse)
        assert_bf16_close("dq", dq[b:b + 1, hs], rdq)
        assert_bf16_close("dk", dk[b:b + 1, hkv:hkv + 1], rdk)
        assert_bf16_close("dv", dv[b:b + 1, hkv:hkv + 1], rdv)
