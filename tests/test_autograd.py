"""GPU: `attention`, the autograd wrapper of attn_fwd / attn_bwd.

Its forward must be attn_fwd's output bit for bit, its gradients attn_bwd's for the same
incoming gradient, and both within the parity bar of the fp64 oracle."""

import pytest
import torch

import exact_attention_27_amd as ea
import oracle
import workloads
from helpers import assert_bf16_close, f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 4, 2, 300, 128), (2, 2, 2, 129, 64)], ids=lambda s: "B%dHq%dHkv%dS%dd%d" % s)
def test_attention_autograd(shape, causal):
    B, Hq, Hkv, S, d = shape
    print(f"\n[autograd] {shape} causal={causal}", flush=True)
    t = workloads.make_tensors(B, Hq, Hkv, S, d, seed=600 + S + d)
    q, k, v, w = (t[n].to(DEV) for n in ("q", "k", "v", "do"))
    qg, kg, vg = (x.clone().requires_grad_(True) for x in (q, k, v))
    o, lse = ea.attention(qg, kg, vg, None, causal, return_lse=True)
    (o.float() * w.float()).sum().backward()  # dL/dO = w (bf16, exactly)
    o_ref, lse_ref = ea.attn_fwd(q, k, v, None, causal)
    dq, dk, dv = ea.attn_bwd(q, k, v, o_ref, lse_ref, w, None, causal)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref) and torch.equal(lse, lse_ref)
    assert torch.equal(qg.grad, dq) and torch.equal(kg.grad, dk) and torch.equal(vg.grad, dv)
    rdq, rdk, rdv = oracle.attention_backward(f64(q), f64(k), f64(v), f64(w), d ** -0.5, causal)
    assert_bf16_close("dq", qg.grad, rdq)
    assert_bf16_close("dk", kg.grad, rdk)
    assert_bf16_close("dv", vg.grad, rdv)


def test_attention_expanded_gradient():
    """out.sum().backward() hands in an expanded (stride 0) gradient of ones."""
    B, Hq, Hkv, S, d = 1, 2, 1, 200, 64
    t = workloads.make_tensors(B, Hq, Hkv, S, d, seed=610)
    q, k, v = (t[n].to(DEV).requires_grad_(True) for n in ("q", "k", "v"))
    ea.attention(q, k, v, causal=True).sum().backward()
    ones = torch.ones(B, Hq, S, d, dtype=torch.bfloat16, device=DEV)
    o, lse = ea.attn_fwd(q.detach(), k.detach(), v.detach(), None, True)
    dq, dk, dv = ea.attn_bwd(q.detach(), k.detach(), v.detach(), o, lse, ones, None, True)
    torch.cuda.synchronize()
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)
    # With dO = 1, sum_j dV_j = G S in every column (each query's probabilities sum to 1),
    # and sum_j dK_j = 0 (each row of dS sums to 0) up to the bf16 rounding of dK.
    G = Hq // Hkv
    assert torch.allclose(dv.float().sum(dim=2), torch.full((B, Hkv, d), float(G * S), device=DEV), rtol=2e-2)
    dkf = dk.float()
    assert (dkf.sum(dim=2).abs() <= 2e-2 * dkf.abs().sum(dim=2) + 1e-3).all()
