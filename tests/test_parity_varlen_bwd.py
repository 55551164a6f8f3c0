"""GPU parity of the packed variable-length backward (attn_bwd_varlen) against the fp64
oracle, sequence by sequence.  Each sequence of a packed batch is an independent
attention problem on its own rows (the packed batches of the hyper.ai FlashAttention-4
story's integration targets), and its gradients are those of the dense backward ("NVIDIA
Blackwell: FlashAttention-4 Overcomes Memory Bottlenecks", body paragraph: the backward
of the same exact attention), so the oracle's head_backward on a sequence's rows is the
reference.  As in the dense tests, the backward consumes the GPU forward's O and LSE
(attn_fwd_varlen), and dK and dV of a KV head are the sums over its query heads.

Small cases: every element of dq, dk and dv of every sequence, ragged lengths including
empty and one-token sequences and lengths on both sides of the 32/64/128-row tiles, MHA
and GQA, d = 64 and 128, causal or not, both dK/dV workgroup shapes.  Also: a batch of
equal-length sequences is bit for bit the dense backward; rows outside every sequence
(and past max_seqlen) are not written.  Full size: the 32-prompt prefill mix, every
element of one KV group's gradients.
"""

import numpy as np
import pytest
import torch

import exact_attention_27_amd as ea
import oracle
import workloads
from helpers import assert_bf16_close, f64
from oracle_pool import Pool, f32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENTINEL = 12288.0  # exact in bf16, and a value no gradient here takes


def run(lengths, Hq, Hkv, d, causal, seed, max_seqlen=None, tail=0, variant=None):
    """Forward then backward of a packed batch on the GPU; the gradients start as SENTINEL."""
    t = workloads.make_varlen_tensors(list(lengths) + ([tail] if tail else []), Hq, Hkv, d, seed, with_do=True)
    cu = t["cu_seqlens"][: len(lengths) + 1].clone()  # a tail of tokens past the last sequence
    dev = {n: x.to(DEV) for n, x in t.items()}
    cud = cu.to(DEV)
    ms = max(lengths, default=0) if max_seqlen is None else max_seqlen
    scale = d ** -0.5
    o, lse = ea.attn_fwd_varlen(dev["q"], dev["k"], dev["v"], cud, ms, scale, causal)
    dq = torch.full_like(dev["q"], SENTINEL)
    dk = torch.full_like(dev["k"], SENTINEL)
    dv = torch.full_like(dev["v"], SENTINEL)
    ea.attn_bwd_varlen(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], cud, ms, scale, causal,
                       dq=dq, dk=dk, dv=dv, variant=variant)
    torch.cuda.synchronize()
    return t, cu, (dq.cpu(), dk.cpu(), dv.cpu()), scale


def oracle_grads(t, cu, Hq, Hkv, scale, causal, max_rows=None, kv_heads=None, pool=False):
    """Per sequence and query head: the oracle's (dq, dk, dv) of that head, with the rows
    they cover (pool: in worker processes, for full-size sequences)."""
    G = Hq // Hkv
    kv_heads = range(Hkv) if kv_heads is None else kv_heads
    tasks, keys = [], []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        n = b - a if max_rows is None else min(b - a, max_rows)
        if n <= 0:
            continue
        for hk in kv_heads:
            for g in range(G):
                h = hk * G + g
                tasks.append((f32(t["q"][a:a + n, h]), f32(t["k"][a:a + n, hk]), f32(t["v"][a:a + n, hk]),
                              f32(t["do"][a:a + n, h]), scale, causal))
                keys.append((a, n, hk, h))
    if pool:
        with Pool() as p:
            res = p.backward(tasks)
    else:
        res = [oracle.head_backward(*x) for x in tasks]
    return keys, res


def check(t, cu, grads, Hq, Hkv, scale, causal, max_rows=None, kv_heads=None, pool=False):
    """Every element of the gradients against the oracle; dk and dv of a KV head are the
    sums of its query heads' oracle gradients."""
    dq, dk, dv = grads
    keys, res = oracle_grads(t, cu, Hq, Hkv, scale, causal, max_rows, kv_heads, pool)
    G = Hq // Hkv
    gq, rq, gk, rk, gv, rv = [], [], [], [], [], []
    acc = {}
    for (a, n, hk, h), (xq, xk, xv) in zip(keys, res):
        gq.append(dq[a:a + n, h]); rq.append(xq)
        sk, sv = acc.get((a, hk), (0.0, 0.0))
        acc[(a, hk)] = (sk + xk, sv + xv)
        if h % G == G - 1:
            gk.append(dk[a:a + n, hk]); rk.append(acc[(a, hk)][0])
            gv.append(dv[a:a + n, hk]); rv.append(acc[(a, hk)][1])
    if not gq:
        return
    assert_bf16_close("dq", torch.cat(gq), np.concatenate(rq))
    assert_bf16_close("dk", torch.cat(gk), np.concatenate(rk))
    assert_bf16_close("dv", torch.cat(gv), np.concatenate(rv))


# (A batch of one single-token sequence is checked exactly below: its dV is the sum of the
# group's dO rows, whose own bf16 rounding alone averages above the mean bar when G = 4.)
LENGTHS = [
    [1, 40], [17], [128], [129, 64], [0, 5, 0, 300, 1], [127, 128, 129, 1, 63, 65, 257, 0],
    [1000, 3, 511, 2],
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,Hq,Hkv", [(64, 4, 2), (128, 4, 1), (128, 2, 2)])
@pytest.mark.parametrize("lengths", LENGTHS, ids=lambda l: "L" + "_".join(map(str, l)))
def test_varlen_bwd_ragged(lengths, d, Hq, Hkv, causal):
    print(f"\n[varlen bwd] lengths={lengths} d={d} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
    t, cu, grads, scale = run(lengths, Hq, Hkv, d, causal, seed=sum(lengths) + d + Hq + 1)
    check(t, cu, grads, Hq, Hkv, scale, causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,Hq,Hkv", [(64, 4, 2), (128, 4, 1)])
def test_single_token_sequences(d, Hq, Hkv, causal):
    """A sequence of one token sees only its own key: P = 1, so dS = P (dP - D) = 0, dQ and
    dK vanish, and dV is the sum of the group's dO rows, correctly rounded to bf16 (to
    within the fp32 rounding of that sum)."""
    lengths = [1, 0, 1, 1]
    print(f"\n[varlen bwd single tokens] d={d} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
    t, cu, (dq, dk, dv), scale = run(lengths, Hq, Hkv, d, causal, seed=61 + d)
    G = Hq // Hkv
    for a in (0, 1, 2):
        assert dq[a].float().abs().max() <= 1e-5 and dk[a].float().abs().max() <= 1e-5
        for hk in range(Hkv):
            ref = t["do"][a, hk * G:(hk + 1) * G].double().sum(0)
            half_ulp = torch.exp2(torch.floor(torch.log2(ref.abs().clamp_min(1e-30))) - 8.0)
            assert ((dv[a, hk].double() - ref).abs() <= half_ulp + 1e-6).all()


@pytest.mark.parametrize("variant", [ea.ATTN_VARIANT_PINGPONG, ea.ATTN_VARIANT_FOURWAVE])
@pytest.mark.parametrize("exp_mode", [ea.ATTN_EXP_HW, ea.ATTN_EXP_POLY3])
def test_varlen_bwd_schedules(variant, exp_mode):
    """Both dK/dV workgroup shapes (eight waves, one per CU; four waves, two per CU) and
    both exponentials, at d = 128 with GQA (the cubic exponential always runs eight)."""
    lengths = [200, 0, 77, 450, 64]
    print(f"\n[varlen bwd schedules] variant={variant} exp_mode={exp_mode}", flush=True)
    t = workloads.make_varlen_tensors(lengths, 4, 2, 128, 93, with_do=True)
    dev = {n: x.to(DEV) for n, x in t.items()}
    ms, scale = max(lengths), 128 ** -0.5
    o, lse = ea.attn_fwd_varlen(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], ms, scale, True, exp_mode=exp_mode)
    dq, dk, dv = ea.attn_bwd_varlen(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], dev["cu_seqlens"], ms, scale,
                                    True, exp_mode=exp_mode, variant=variant)
    torch.cuda.synchronize()
    check(t, t["cu_seqlens"], (dq.cpu(), dk.cpu(), dv.cpu()), 4, 2, scale, True)


def to_dense(x, nseq, S):
    """[nseq*S, H, d] packed rows of equal-length sequences as the dense [nseq, H, S, d]."""
    return x.reshape(nseq, S, x.shape[1], x.shape[2]).permute(0, 2, 1, 3).contiguous()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,Hq,Hkv,variant", [(64, 4, 2, None), (128, 8, 2, ea.ATTN_VARIANT_PINGPONG),
                                              (128, 4, 4, ea.ATTN_VARIANT_FOURWAVE)])
def test_equal_lengths_are_the_dense_backward(d, Hq, Hkv, variant, causal):
    """nseq sequences of one length S give the dense [nseq, H, S, d] backward's bits: the
    packed kernels run the same arithmetic in the same order, only their rows live elsewhere."""
    nseq, S = 3, 333
    print(f"\n[varlen bwd == dense] nseq={nseq} S={S} d={d} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
    t, cu, (dq, dk, dv), scale = run([S] * nseq, Hq, Hkv, d, causal, seed=40 + d + Hq, variant=variant)
    q, k, v, do = (to_dense(t[n], nseq, S).to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = ea.attn_fwd(q, k, v, scale, causal)
    rq, rk, rv = ea.attn_bwd_ex(q, k, v, o, lse, do, scale, causal, variant=variant)
    torch.cuda.synchronize()
    assert torch.equal(to_dense(dq, nseq, S), rq.cpu())
    assert torch.equal(to_dense(dk, nseq, S), rk.cpu())
    assert torch.equal(to_dense(dv, nseq, S), rv.cpu())


def test_rows_outside_the_sequences_are_left_alone():
    """Tokens past cu_seqlens[nseq], and rows of a sequence past max_seqlen, get no
    gradient written; a sequence longer than max_seqlen is taken as its first max_seqlen
    rows (causal: those rows' forward already saw only them)."""
    Hq, Hkv, d = 4, 2, 64
    lengths = [300, 90]
    print("\n[varlen bwd unwritten rows]", flush=True)
    t, cu, (dq, dk, dv), scale = run(lengths, Hq, Hkv, d, True, seed=19, max_seqlen=200, tail=40)
    for r in list(range(200, 300)) + list(range(390, 430)):
        for x in (dq, dk, dv):
            assert (x[r].float() == SENTINEL).all(), r
    check(t, cu, (dq, dk, dv), Hq, Hkv, scale, True, max_rows=200)


def test_varlen_bwd_prefill_workload():
    """The 32-prompt prefill mix at full size (GQA 32:8, d = 128, causal), in the launch
    configuration bench.py times: every element of KV group 0's gradients (its 4 query
    heads' dq, and dk and dv) in every sequence, and the other groups' gradients finite."""
    w = workloads.VARLEN_WORKLOADS[9]
    print(f"\n[varlen bwd workload] {w.describe()}", flush=True)
    host = workloads.make_varlen_inputs(w, with_do=True)
    dev = {n: x.to(DEV) for n, x in host.items()}
    ms = max(w.lengths())
    o, lse = ea.attn_fwd_varlen(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], ms, w.scale, w.causal)
    dq, dk, dv = ea.attn_bwd_varlen(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], dev["cu_seqlens"], ms, w.scale,
                                    w.causal)
    torch.cuda.synchronize()
    for x in (dq, dk, dv):
        assert torch.isfinite(x.float()).all()
    check(host, host["cu_seqlens"], (dq.cpu(), dk.cpu(), dv.cpu()), w.Hq, w.Hkv, w.scale, w.causal, kv_heads=[0],
          pool=True)


@pytest.mark.parametrize("causal", [False, True])
def test_offsets_outside_the_tensor_are_clamped(causal):
    """cu_seqlens entries below 0 or past total are clamped (include/attn.h): offsets
    [-7, 40, 40, 130] over 100 tokens are the sequences [0, 40), [40, 40) (empty) and
    [40, 100).  Both packed passes compute exactly those sequences."""
    Hq, Hkv, d, total = 4, 2, 64, 100
    print(f"\n[varlen clamped offsets] causal={causal}", flush=True)
    t = workloads.make_varlen_tensors([total], Hq, Hkv, d, 71, with_do=True)
    dev = {n: x.to(DEV) for n, x in t.items()}
    cu = torch.tensor([-7, 40, 40, 130], dtype=torch.int32, device=DEV)
    scale = d ** -0.5
    o, lse = ea.attn_fwd_varlen(dev["q"], dev["k"], dev["v"], cu, 60, scale, causal)
    dq, dk, dv = ea.attn_bwd_varlen(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], cu, 60, scale, causal)
    torch.cuda.synchronize()
    G = Hq // Hkv
    real = torch.tensor([0, 40, 40, 100], dtype=torch.int32)
    for s in range(3):
        a, b = int(real[s]), int(real[s + 1])
        for h in range(Hq):
            x, y = oracle.head_forward(f64(t["q"][a:b, h]), f64(t["k"][a:b, h // G]), f64(t["v"][a:b, h // G]),
                                       scale, causal)
            if b > a:
                assert_bf16_close("o", o[a:b, h].cpu(), x)
                assert np.abs(f64(lse[h, a:b]) - y).max() <= 1e-3
    check(t, real, (dq.cpu(), dk.cpu(), dv.cpu()), Hq, Hkv, scale, causal)
