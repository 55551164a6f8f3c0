"""GPU robustness: the forward and backward captured in a HIP graph and replayed (the
library allocates nothing and issues no memset, so a capture records only its kernels);
many small heads (a large grid of one-tile workgroups); and a packed batch of hundreds of
sequences.  Parity against the fp64 oracle or bitwise against eager launches.
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


def test_graph_capture_and_replay():
    """fwd + bwd captured once on a side stream, replayed three times with eager work and
    synchronizations between replays; every replay equals the eager result bit for bit."""
    B, Hq, Hkv, S, d = 2, 8, 2, 700, 128
    print(f"\n[graph] B={B} Hq={Hq} Hkv={Hkv} S={S} d={d}", flush=True)
    t = {n: x.to(DEV) for n, x in workloads.make_tensors(B, Hq, Hkv, S, d, seed=41).items()}
    scale = d ** -0.5
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], scale, True)
    dq, dk, dv = ea.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], scale, True)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (o, lse, dq, dk, dv)]

    go, glse = torch.empty_like(o), torch.empty_like(lse)
    gdq, gdk, gdv = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(B, Hq, Hkv, S, d), dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        ea.attn_fwd(t["q"], t["k"], t["v"], scale, True, o=go, lse=glse)
        ea.attn_bwd_ex(t["q"], t["k"], t["v"], go, glse, t["do"], scale, True, gdq, gdk, gdv, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ea.attn_fwd(t["q"], t["k"], t["v"], scale, True, o=go, lse=glse)
        ea.attn_bwd_ex(t["q"], t["k"], t["v"], go, glse, t["do"], scale, True, gdq, gdk, gdv, ws)
    for rep in range(3):
        for x in (go, glse, gdq, gdk, gdv):
            x.fill_(float("nan") if x.dtype == torch.float32 else 7.0)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(("o", "lse", "dq", "dk", "dv"), (go, glse, gdq, gdk, gdv), ref):
            assert torch.equal(x, r), f"replay {rep}: {name} differs from the eager result"


def test_packed_graph_capture_and_replay():
    """The packed forward and backward captured once, replayed three times with eager work
    between replays; every replay equals the eager result bit for bit (the library
    allocates nothing, and the caller hands in the workspace)."""
    lengths, Hq, Hkv, d = [300, 1, 0, 517, 64], 8, 2, 128
    print(f"\n[packed graph] lengths={lengths} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    t = {n: x.to(DEV) for n, x in workloads.make_varlen_tensors(lengths, Hq, Hkv, d, 43, with_do=True).items()}
    cu, ms, scale = t["cu_seqlens"], max(lengths), d ** -0.5
    o, lse = ea.attn_fwd_varlen(t["q"], t["k"], t["v"], cu, ms, scale, True)
    dq, dk, dv = ea.attn_bwd_varlen(t["q"], t["k"], t["v"], o, lse, t["do"], cu, ms, scale, True)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (o, lse, dq, dk, dv)]

    go, glse = torch.empty_like(o), torch.empty_like(lse)
    gdq, gdk, gdv = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    ws = torch.empty(ea.attn_bwd_varlen_workspace_bytes(len(lengths), int(t["q"].shape[0]), Hq, Hkv, d),
                     dtype=torch.uint8, device=DEV)

    def passes():
        ea.attn_fwd_varlen(t["q"], t["k"], t["v"], cu, ms, scale, True, o=go, lse=glse)
        ea.attn_bwd_varlen(t["q"], t["k"], t["v"], go, glse, t["do"], cu, ms, scale, True, gdq, gdk, gdv, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        passes()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        passes()
    for rep in range(3):
        for x in (go, glse, gdq, gdk, gdv):
            x.fill_(float("nan") if x.dtype == torch.float32 else 7.0)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(("o", "lse", "dq", "dk", "dv"), (go, glse, gdq, gdk, gdv), ref):
            assert torch.equal(x, r), f"replay {rep}: {name} differs from the eager result"


def test_many_small_heads():
    """A large grid of short sequences: B=96, Hq=16, Hkv=4, S=100 (one query tile and two
    key tiles per head, the last one ragged); sampled heads against the oracle."""
    B, Hq, Hkv, S, d = 96, 16, 4, 100, 64
    print(f"\n[many heads] B={B} Hq={Hq} Hkv={Hkv} S={S} d={d}", flush=True)
    host = workloads.make_tensors(B, Hq, Hkv, S, d, seed=43)
    t = {n: x.to(DEV) for n, x in host.items()}
    scale = d ** -0.5
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], scale, True)
    dq, dk, dv = ea.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], scale, True)
    torch.cuda.synchronize()
    G = Hq // Hkv
    picks = [(0, 0), (17, 5), (50, 11), (95, 15)]
    for b, h in picks:
        q, k, v, do = (f64(host[n][b, h if n in ("q", "do") else h // G]) for n in ("q", "k", "v", "do"))
        ro, rl = oracle.head_forward(q, k, v, scale, True)
        assert_bf16_close(f"o[{b},{h}]", o[b, h], ro)
        assert_lse_close(lse[b, h], rl)
    # dK/dV are sums over the group: check one whole group with the oracle
    b, hk = 33, 2
    gk, gv = np.zeros((S, d)), np.zeros((S, d))
    for g in range(G):
        h = hk * G + g
        rq, rk, rv = oracle.head_backward(f64(host["q"][b, h]), f64(host["k"][b, hk]), f64(host["v"][b, hk]),
                                          f64(host["do"][b, h]), scale, True)
        assert_bf16_close(f"dq[{b},{h}]", dq[b, h], rq)
        gk += rk
        gv += rv
    assert_bf16_close("dk group", dk[b, hk], gk)
    assert_bf16_close("dv group", dv[b, hk], gv)


def test_varlen_many_sequences():
    """300 sequences of seeded lengths in 0..400 (many empty or shorter than a tile);
    every sequence checked on sampled rows of two heads."""
    g = np.random.default_rng(45)
    lengths = [int(x) for x in g.integers(0, 401, size=300)]
    lengths[:5] = [0, 1, 0, 400, 128]
    Hq, Hkv, d = 4, 1, 128
    print(f"\n[varlen many] {len(lengths)} sequences, total {sum(lengths)}", flush=True)
    t = workloads.make_varlen_tensors(lengths, Hq, Hkv, d, seed=46)
    dev = {n: x.to(DEV) for n, x in t.items()}
    o, lse = ea.attn_fwd_varlen(dev["q"], dev["k"], dev["v"], dev["cu_seqlens"], max(lengths), None, True)
    torch.cuda.synchronize()
    og, lg = o.cpu(), lse.cpu()
    cu = t["cu_seqlens"].tolist()
    go, gl, ro, rl = [], [], [], []
    for s, n in enumerate(lengths):
        if n == 0:
            continue
        a = cu[s]
        rows = np.unique(np.array([0, n // 2, n - 1]))
        for h in (0, 3):
            x, y = oracle.head_forward(f64(t["q"][a:a + n, h]), f64(t["k"][a:a + n, 0]), f64(t["v"][a:a + n, 0]),
                                       d ** -0.5, True, rows=rows)
            go.append(og[a + rows, h]); gl.append(lg[h, a + rows]); ro.append(x); rl.append(y)
    assert_bf16_close("o", torch.cat(go), np.concatenate(ro))
    assert_lse_close(torch.cat(gl), np.concatenate(rl))
