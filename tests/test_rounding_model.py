"""The rounding model (tests/rounding_model.py) on the case that decides how the backward
forms the row term D (CPU only).

With eight query heads per KV head on a short causal sequence, the first keys gather
probability from every row of all eight heads, so dK there is most sensitive to an error
in D.  The backward's dK/dV products use D_i = sum_j P_ij dP_ij, which the dQ pass forms
(the gradient formulas of exact attention; see the oracle).  The alternative, taking D_i
from the stored bf16 O as <dO_i, O_i>, is what a backward that accumulates dQ inside the
dK/dV pass (no second pass over the keys before dK) would have to use: with it the model
puts dK within a few percent of the max-abs 2e-2 bar, with no room left for the fp32
accumulation the GPU adds.  These tests pin both numbers, so a change of the kernels'
roundings that the model describes shows up here first.
"""

import numpy as np

import oracle
import rounding_model as rm
import workloads
from helpers import f64, parity_bound


def margins(case, causal, **kw):
    """Largest |model - oracle| / bar over each gradient."""
    B, Hq, Hkv, S, d = case
    t = workloads.make_tensors(B, Hq, Hkv, S, d, 100 + sum(case))
    q, k, v, do = (f64(t[n]) for n in ("q", "k", "v", "do"))
    scale = d ** -0.5
    ref = oracle.attention_backward(q, k, v, do, scale, causal)
    _, _, *model = rm.attention(q, k, v, do, scale, causal, **kw)
    return [float((np.abs(m - r) / parity_bound(r)).max()) for m, r in zip(model, ref)]


MQA = (1, 8, 1, 200, 64)  # the backward edge case of the GPU tests with eight heads per KV head


def test_exact_row_term_leaves_room():
    dq, dk, dv = margins(MQA, True)
    assert dk < 0.8 and dq < 0.8 and dv < 0.85, (dq, dk, dv)


def test_row_term_from_bf16_output_reaches_the_bar():
    exact = margins(MQA, True)[1]
    from_o = margins(MQA, True, dkv_d_from_o=True)[1]
    assert from_o > 0.95 and from_o > exact + 0.2, (exact, from_o)


def test_bf16_probabilities_in_dv_exceed_the_bar():
    """bf16 P in dV^T += dO^T P (the kernels use fp16 P) puts dV over the bar on this case."""
    assert margins(MQA, True)[2] < 0.85
    assert margins(MQA, True, p_fmt="bf16")[2] > 1.0
