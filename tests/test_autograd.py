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


@pytest.mark.parametrize("causal", [False, True])
def test_attention_varlen_autograd(causal):
    """attention_varlen: the forward is attn_fwd_varlen's bit for bit, the gradients
    attn_bwd_varlen's for the same incoming gradient, rows past the last sequence get a
    zero gradient, and each sequence's gradients meet the parity bar of the oracle."""
    lengths, Hq, Hkv, d = [150, 1, 0, 333], 4, 2, 128
    print(f"\n[autograd varlen] lengths={lengths} causal={causal}", flush=True)
    t = workloads.make_varlen_tensors(lengths + [7], Hq, Hkv, d, seed=620, with_do=True)  # 7 tail tokens
    cu = t["cu_seqlens"][: len(lengths) + 1].to(DEV)
    q, k, v, w = (t[n].to(DEV) for n in ("q", "k", "v", "do"))
    ms = max(lengths)
    qg, kg, vg = (x.clone().requires_grad_(True) for x in (q, k, v))
    o, lse = ea.attention_varlen(qg, kg, vg, cu, ms, None, causal, return_lse=True)
    (o.float() * w.float()).sum().backward()
    o_ref, lse_ref = ea.attn_fwd_varlen(q, k, v, cu, ms, None, causal)
    dq, dk, dv = ea.attn_bwd_varlen(q, k, v, o_ref, lse_ref, w, cu, ms, None, causal)
    torch.cuda.synchronize()
    n = sum(lengths)
    assert torch.equal(o.detach()[:n], o_ref[:n]) and torch.equal(lse[:, :n], lse_ref[:, :n])
    assert torch.equal(qg.grad[:n], dq[:n]) and torch.equal(kg.grad[:n], dk[:n]) and torch.equal(vg.grad[:n], dv[:n])
    for g in (qg.grad, kg.grad, vg.grad):
        assert (g[n:] == 0).all()
    G, a = Hq // Hkv, 0
    for L in lengths:
        if L:
            x = [f64(t[nm][a:a + L]).transpose(1, 0, 2)[None] for nm in ("q", "k", "v", "do")]
            rdq, rdk, rdv = oracle.attention_backward(*x, d ** -0.5, causal)
            assert_bf16_close("dq", qg.grad[a:a + L].transpose(0, 1)[None], rdq)
            assert_bf16_close("dk", kg.grad[a:a + L].transpose(0, 1)[None], rdk)
            if L > 1:  # (a one-token sequence's dV is checked exactly in the packed backward's tests)
                assert_bf16_close("dv", vg.grad[a:a + L].transpose(0, 1)[None], rdv)
        a += L
