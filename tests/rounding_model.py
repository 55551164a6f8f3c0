"""CPU model of the roundings the GPU kernels make, for explaining their errors.

Test infrastructure only (like the oracle; nothing in the product imports it).  It is
not a second oracle: it takes the textbook attention of the fp64 oracle and inserts, one
switch at a time, the points where the kernels round to a narrower format.  Each rounding
is applied where the kernels apply it; everything else is done in float64.  Comparing the
model with the oracle tells how much of a GPU error each rounding explains, and which
kernel change removes it.

Rounding points (names in ``on``):
  fwd_p    the forward rounds each probability 2^(x - m_ref) to bf16 before the P.V
           product (the running sum adds the unrounded values); m_ref follows the
           tile-wise rescale rule (tau = 8, 64-key tiles, a rescale moves every row of
           the 32-row wave).
  out      every bf16 output (O, dQ, dK, dV) is rounded to nearest even.
  bwd_o    the dQ kernel's row term D_i = <dO_i, O_i> uses the stored bf16 O (from the
           model's own forward).  With ``dkv_d_from_o`` the dK/dV products use that D
           too (the earlier kernels); otherwise they use D_i = sum_j P_ij dP_ij, which
           the dQ kernel now forms from the dS row sums.
  bwd_p    the backward rounds P for dV^T += dO^T P, to ``p_fmt`` ("fp16", the current
           kernels, whose dO operand is scaled into fp16 exactly; "bf16" before).
  bwd_ds   the backward rounds dS for dK^T += Q^T dS, to ``dsk_fmt`` ("fp16", the current
           kernels, whose Q operand is scaled into fp16 exactly; "bf16" before), and to
           bf16 for dQ^T += K^T dS^T.
"""

from __future__ import annotations

import numpy as np

ALL = ("fwd_p", "out", "bwd_o", "bwd_p", "bwd_ds")


def bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isfinite(f), out, f.astype(np.float64))


def fp16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest fp16 (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def head_forward(q, k, v, scale, causal, on=ALL, tau=8.0, bn=64):
    """Forward of one head with the chosen roundings: (o, lse), float64."""
    S, d = q.shape
    c = scale * np.log2(np.e)
    x = (q @ k.T) * c  # log2 units
    if causal:
        x[np.arange(S)[None, :] > np.arange(S)[:, None]] = -np.inf
    m_ref = np.full(S, -np.inf)
    l = np.zeros(S)
    acc = np.zeros((S, d))
    for k0 in range(0, S, bn):
        xt = x[:, k0:k0 + bn]
        mt = xt.max(axis=1)
        grow = mt > m_ref + tau
        # The rule is applied per wave of 32 rows: a row over the threshold rescales its
        # whole wave, every row of which then takes max(m_ref, tile maximum).
        for w0 in range(0, S, 32):
            sl = slice(w0, w0 + 32)
            if grow[sl].any():
                m_new = np.maximum(m_ref[sl], mt[sl])
                alpha = np.where(m_new == -np.inf, 1.0, np.exp2(m_ref[sl] - m_new))
                acc[sl] *= alpha[:, None]
                l[sl] *= alpha
                m_ref[sl] = m_new
        mr = np.where(m_ref == -np.inf, 0.0, m_ref)
        p = np.exp2(xt - mr[:, None])
        l += p.sum(axis=1)
        pr = bf16(p) if "fwd_p" in on else p
        acc += pr @ v[k0:k0 + bn]
    o = acc / l[:, None]
    lse = (m_ref + np.log2(l)) * np.log(2.0)
    return (bf16(o) if "out" in on else o), lse


def head_backward(q, k, v, do, o, lse, scale, causal, on=ALL, p_fmt="fp16", dkv_d_from_o=False, dsk_fmt="fp16"):
    """Backward of one head from the given o and lse: (dq, dk, dv) float64, before output
    rounding (the caller rounds after any group sum)."""
    S, d = q.shape
    s = scale * (q @ k.T)
    if causal:
        s[np.arange(S)[None, :] > np.arange(S)[:, None]] = -np.inf
    p = np.exp(s - lse[:, None])
    dp = do @ v.T
    d_o = (do * o).sum(axis=1)    # D from the O given (bf16 when "bwd_o")
    d_x = (p * dp).sum(axis=1)    # D from its definition
    ds_q = p * (dp - d_o[:, None])
    ds_kv = ds_q if dkv_d_from_o else p * (dp - d_x[:, None])
    rnd_p = {"fp16": fp16, "bf16": bf16}[p_fmt]
    pr = rnd_p(p) if "bwd_p" in on else p
    if "bwd_ds" in on:
        ds_q, ds_kv = bf16(ds_q), {"fp16": fp16, "bf16": bf16}[dsk_fmt](ds_kv)
    return scale * (ds_q @ k), scale * (ds_kv.T @ q), pr.T @ do


def attention(q, k, v, do, scale, causal, on=ALL, p_fmt="fp16", dkv_d_from_o=False, dsk_fmt="fp16"):
    """Whole problem [B,H,S,d] through the model: (o, lse, dq, dk, dv), float64."""
    from oracle import head_forward as exact_forward

    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = np.empty_like(q)
    lse = np.empty((B, Hq, S))
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            oh, lh = head_forward(q[b, h], k[b, hk], v[b, hk], scale, causal, on)
            o[b, h], lse[b, h] = oh, lh
            if "bwd_o" in on:
                ob = bf16(oh)  # the only O the backward has
            else:
                ob, lh = exact_forward(q[b, h], k[b, hk], v[b, hk], scale, causal)
            a, bb, cc = head_backward(q[b, h], k[b, hk], v[b, hk], do[b, h], ob, lh, scale, causal, on,
                                      p_fmt, dkv_d_from_o, dsk_fmt)
            dq[b, h] = a
            dk[b, hk] += bb
            dv[b, hk] += cc
    r = bf16 if "out" in on else (lambda x: x)
    return o, lse, r(dq), r(dk), r(dv)
