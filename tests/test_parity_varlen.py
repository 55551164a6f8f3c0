"""GPU parity of the packed variable-length forward (attn_fwd_varlen) against the fp64
oracle, sequence by sequence: every sequence of a packed batch is an independent
attention problem on its own rows (the prefill batches of SGLang and vLLM that the hyper.ai
FlashAttention-4 story names as FA4's integration target hold prompts of different
lengths; the pages give no interface, so a packed batch only changes where each
sequence's rows live).

Small cases: the oracle on every row of every (sequence, head), with ragged lengths
including empty and one-token sequences and lengths on both sides of the 64-key and
128-query tiles.  Full size (the 32-prompt prefill mix): all heads, sampled rows per
sequence.  Also: a single packed sequence is bit for bit the dense forward, and rows
that no sequence covers (or that lie past max_seqlen) are left as they were.
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
SENTINEL = 12288.0  # exact in bf16, and a value no output here takes (|O| <= max |V| < 10)


def run(lengths, Hq, Hkv, d, causal, seed, max_seqlen=None, tail=0, **kw):
    t = workloads.make_varlen_tensors(list(lengths) + ([tail] if tail else []), Hq, Hkv, d, seed)
    cu = t["cu_seqlens"][: len(lengths) + 1].clone()  # a tail of tokens past the last sequence
    dev = {n: x.to(DEV) for n, x in t.items()}
    total = int(t["q"].shape[0])
    o = torch.full((total, Hq, d), SENTINEL, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((Hq, total), SENTINEL, dtype=torch.float32, device=DEV)
    ms = max(lengths, default=0) if max_seqlen is None else max_seqlen
    scale = d ** -0.5
    ea.attn_fwd_varlen(dev["q"], dev["k"], dev["v"], cu.to(DEV), ms, scale, causal, o=o, lse=lse, **kw)
    torch.cuda.synchronize()
    return t, cu, o.cpu(), lse.cpu(), scale


def check_all_rows(t, cu, o, lse, Hq, Hkv, scale, causal, max_rows=None):
    G = Hq // Hkv
    go, gl, ro, rl = [], [], [], []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        n = b - a if max_rows is None else min(b - a, max_rows)
        if n <= 0:
            continue
        for h in range(Hq):
            q = f64(t["q"][a:b, h]); k = f64(t["k"][a:b, h // G]); v = f64(t["v"][a:b, h // G])
            x, y = oracle.head_forward(q, k, v, scale, causal, rows=np.arange(n))
            go.append(o[a:a + n, h]); gl.append(lse[h, a:a + n]); ro.append(x); rl.append(y)
    assert_bf16_close("o", torch.cat(go), np.concatenate(ro))
    assert_lse_close(torch.cat(gl), np.concatenate(rl))


LENGTHS = [
    [1], [17], [128], [129, 64], [0, 5, 0, 300, 1], [127, 128, 129, 1, 63, 65, 257, 0],
    [1000, 3, 511, 2],
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,Hq,Hkv", [(64, 4, 2), (128, 4, 1), (128, 2, 2)])
@pytest.mark.parametrize("lengths", LENGTHS, ids=lambda l: "L" + "_".join(map(str, l)))
def test_varlen_ragged(lengths, d, Hq, Hkv, causal):
    print(f"\n[varlen] lengths={lengths} d={d} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
    t, cu, o, lse, scale = run(lengths, Hq, Hkv, d, causal, seed=sum(lengths) + d + Hq)
    check_all_rows(t, cu, o, lse, Hq, Hkv, scale, causal)
    if causal:  # the first query of a sequence sees only its own key: O is V bit for bit
        G = Hq // Hkv
        for s in range(len(lengths)):
            a = int(cu[s])
            if lengths[s] > 0:
                for h in range(Hq):
                    assert torch.equal(o[a, h], t["v"][a, h // G])


@pytest.mark.parametrize("exp_mode", [ea.ATTN_EXP_HW, ea.ATTN_EXP_POLY3])
@pytest.mark.parametrize("tau", [0.0, 30.0])
def test_varlen_options(exp_mode, tau):
    lengths = [200, 0, 77, 450]
    print(f"\n[varlen options] exp_mode={exp_mode} tau={tau}", flush=True)
    t, cu, o, lse, scale = run(lengths, 4, 2, 128, True, seed=91, exp_mode=exp_mode, tau=tau)
    check_all_rows(t, cu, o, lse, 4, 2, scale, True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_single_sequence_is_the_dense_forward(d, causal):
    """One packed sequence [S, H, d] gives the dense [1, H, S, d] forward's bits."""
    S, Hq, Hkv = 777, 4, 2
    print(f"\n[varlen == dense] S={S} d={d} causal={causal}", flush=True)
    t, cu, o, lse, scale = run([S], Hq, Hkv, d, causal, seed=5 + d)
    q = t["q"].permute(1, 0, 2).unsqueeze(0).contiguous().to(DEV)
    k = t["k"].permute(1, 0, 2).unsqueeze(0).contiguous().to(DEV)
    v = t["v"].permute(1, 0, 2).unsqueeze(0).contiguous().to(DEV)
    od, ld = ea.attn_fwd(q, k, v, scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(o, od[0].permute(1, 0, 2).cpu())
    assert torch.equal(lse, ld[0].cpu())


@pytest.mark.parametrize("causal", [False, True])
def test_rows_outside_the_sequences_are_left_alone(causal):
    """Tokens past cu_seqlens[nseq], and rows of a sequence past max_seqlen, are not
    written; the rows that are written are still right (over all their sequence's keys)."""
    Hq, Hkv, d = 4, 2, 64
    lengths = [300, 90]
    print(f"\n[varlen unwritten rows] causal={causal}", flush=True)
    t, cu, o, lse, scale = run(lengths, Hq, Hkv, d, causal, seed=17, max_seqlen=200, tail=40)
    # rows 200..299 of sequence 0 (past max_seqlen) and the 40-token tail: untouched
    for r in list(range(200, 300)) + list(range(390, 430)):
        assert (o[r].float() == SENTINEL).all() and (lse[:, r] == SENTINEL).all(), r
    assert torch.isfinite(o[:200].float()).all() and torch.isfinite(o[300:390].float()).all()
    check_all_rows(t, cu, o, lse, Hq, Hkv, scale, causal, max_rows=200)


def test_varlen_prefill_workload():
    """The 32-prompt prefill mix at full size (GQA 32:8, d=128, causal), in the launch
    configuration bench.py times: every head of every sequence on sampled rows (fixed
    tile-edge rows plus seeded ones), and the first row of every sequence exactly."""
    w = workloads.VARLEN_WORKLOADS[9]
    print(f"\n[varlen workload] {w.describe()}", flush=True)
    host = workloads.make_varlen_inputs(w)
    dev = {n: x.to(DEV) for n, x in host.items()}
    lens = w.lengths()
    o, lse = ea.attn_fwd_varlen(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], max(lens), w.scale, w.causal)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    og, lg = o.cpu(), lse.cpu()
    cu = host["cu_seqlens"].tolist()
    G = w.group
    g = np.random.default_rng(9000)
    go, gl, ro, rl = [], [], [], []
    for s, n in enumerate(lens):
        a = cu[s]
        fixed = np.array([0, 1, 63, 64, 127, 128, 129, n // 2, n - 2, n - 1])
        for h in range(w.Hq):
            assert torch.equal(og[a, h], host["v"][a, h // G])
            rows = np.unique(np.concatenate([fixed[(fixed >= 0) & (fixed < n)], g.choice(n, size=6, replace=False)]))
            x, y = oracle.head_forward(f64(host["q"][a:a + n, h]), f64(host["k"][a:a + n, h // G]),
                                       f64(host["v"][a:a + n, h // G]), w.scale, w.causal, rows=rows)
            sel = torch.from_numpy(rows + a)
            go.append(og[sel, h]); gl.append(lg[h, sel]); ro.append(x); rl.append(y)
    assert_bf16_close("o", torch.cat(go), np.concatenate(ro))
    assert_lse_close(torch.cat(gl), np.concatenate(rl))
