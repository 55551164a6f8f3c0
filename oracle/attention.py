"""fp64 CPU oracle: exact scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain numpy, no tiling over
keys, no online softmax, no exp2, no approximation.  Nothing here is shared with
the HIP kernels.

What is computed, and where it comes from
-----------------------------------------
The pages describe FlashAttention-4 as an *exact* attention kernel: self-attention
relates every token of the sequence to every other one, at a cost quadratic in the
sequence length, and the method only changes how fast that result is reached
(hyper.ai FlashAttention-4 story, single paragraph; "NVIDIA Blackwell:
FlashAttention-4 Overcomes Memory Bottlenecks", body paragraph).  Both passes are
in scope: the backward pass is named on the same two pages and in section "The chip
is fast; the calculation still waits" of the frontieraireview.com article.  The
pages print no formula, so the oracle is the textbook definition of scaled
dot-product attention with a softmax over keys:

    s_ij   = scale * <q_i, k_j>                      for j in V(i)
    V(i)   = {j : j <= i} if causal else all j       (diagonal included)
    LSE_i  = log sum_{j in V(i)} exp(s_ij)           (natural log)
    P_ij   = exp(s_ij - LSE_i), 0 outside V(i)
    O_i    = sum_j P_ij v_j

and, for a given upstream gradient dO of a scalar loss, the exact derivatives:

    dV_j   = sum_i P_ij dO_i
    dP_ij  = <dO_i, v_j>
    D_i    = sum_j P_ij dP_ij
    dS_ij  = P_ij (dP_ij - D_i)
    dQ_i   = scale * sum_j dS_ij k_j
    dK_j   = scale * sum_i dS_ij q_i

Grouped-query attention (the GQA/MQA head sharing that the ainvest.com article,
section "Limitations and the Road Ahead", lists as missing from FA4): query head
``hq`` reads key/value head ``hq // G`` with ``G = Hq // Hkv``, and the gradients
of a key/value head are the sums over its ``G`` query heads.

Layouts: q, o, do, dq are [B, Hq, S, d]; k, v, dk, dv are [B, Hkv, S, d]; lse is
[B, Hq, S].  Inputs of any real dtype are upcast to float64 first.
"""

from __future__ import annotations

import numpy as np

# Query rows per block.  Blocking over rows only bounds memory (rows x S scores);
# every row still sees all of its keys at once, so the arithmetic per row is the
# plain definition above.
ROW_BLOCK = 512


def kv_head_of(hq: int, Hq: int, Hkv: int) -> int:
    """Key/value head read by query head ``hq``: contiguous groups of G = Hq/Hkv."""
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} must be a positive multiple of Hkv={Hkv}")
    return hq // (Hq // Hkv)


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _scores(q_rows: np.ndarray, k: np.ndarray, rows: np.ndarray, scale: float, causal: bool) -> np.ndarray:
    """s = scale * q_rows k^T with keys outside V(i) set to -inf."""
    s = scale * (q_rows @ k.T)
    if causal:
        keys = np.arange(k.shape[0])
        s[keys[None, :] > rows[:, None]] = -np.inf
    return s


def _softmax_rows(s: np.ndarray):
    """Row softmax of s (with -inf entries) and the natural-log logsumexp of each row."""
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, (m + np.log(l))[:, 0]


def head_forward(q, k, v, scale: float, causal: bool, rows=None):
    """Forward pass of one (batch, query head) pair.

    q: [S, d] queries of this head; k, v: [S, d] keys/values of its KV head.
    rows: optional 1-D array of query positions to evaluate (default: all S).
    Returns (o [R, d], lse [R]) in float64 for the R requested rows.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.shape[0], v.shape[1]))
    lse = np.empty(rows.shape[0])
    for a in range(0, rows.shape[0], ROW_BLOCK):
        r = rows[a:a + ROW_BLOCK]
        p, lse[a:a + r.shape[0]] = _softmax_rows(_scores(q[r], k, r, scale, causal))
        o[a:a + r.shape[0]] = p @ v
    return o, lse


def head_backward(q, k, v, do, scale: float, causal: bool):
    """Backward pass of one (batch, query head) pair, recomputing P from its definition.

    Returns (dq [S, d], dk [S, d], dv [S, d]) in float64; dk and dv are this query
    head's contributions to its KV head's gradients.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    S = q.shape[0]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for a in range(0, S, ROW_BLOCK):
        r = np.arange(a, min(a + ROW_BLOCK, S))
        p, _ = _softmax_rows(_scores(q[r], k, r, scale, causal))
        dp = do[r] @ v.T
        D = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - D)
        dq[r] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r])
        dv += p.T @ do[r]
    return dq, dk, dv


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.shape != v.shape or k.ndim != 4:
        raise ValueError("expected q [B,Hq,S,d] and k, v [B,Hkv,S,d]")
    B, Hq, S, d = q.shape
    if k.shape[0] != B or k.shape[2] != S or k.shape[3] != d:
        raise ValueError("q and k/v disagree on B, S or d")
    kv_head_of(0, Hq, k.shape[1])
    return B, Hq, k.shape[1], S, d


def attention_forward(q, k, v, scale: float, causal: bool):
    """Full forward pass.  Returns (o [B,Hq,S,d], lse [B,Hq,S]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, S, d = _check_shapes(q, k, v)
    o = np.empty((B, Hq, S, d))
    lse = np.empty((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            o[b, h], lse[b, h] = head_forward(q[b, h], k[b, hk], v[b, hk], scale, causal)
    return o, lse


def attention_backward(q, k, v, do, scale: float, causal: bool):
    """Full backward pass.  Returns (dq, dk, dv) in float64; dk, dv summed over each group."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Hkv, S, d = _check_shapes(q, k, v)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            dq[b, h], dkh, dvh = head_backward(q[b, h], k[b, hk], v[b, hk], do[b, h], scale, causal)
            dk[b, hk] += dkh
            dv[b, hk] += dvh
    return dq, dk, dv
