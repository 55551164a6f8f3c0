"""Derive the cubic exp2 polynomial used by the softmax (constants kExp2C1..3 in attn_device.h).

2^x = 2^n * 2^f with n = round(x), f in [-1/2, 1/2].  p(f) = 1 + c1 f + c2 f^2 + c3 f^3
(p(0) = 1 exactly, so integer powers of two are exact) minimises the maximum relative
error max |p(f) / 2^f - 1| over [-1/2, 1/2]: a linear program in (c1, c2, c3, e) on a
dense grid.  The float32-rounded coefficients are printed with their error.

    python exact_attention_27_amd/csrc/fit_exp2_poly.py
"""

import numpy as np
from scipy.optimize import linprog


def fit(deg: int = 3, n: int = 20001):
    f = np.linspace(-0.5, 0.5, n)
    t = 2.0 ** f
    A = np.stack([f ** k / t for k in range(1, deg + 1)], axis=1)
    base = 1.0 / t - 1.0
    ones = np.ones((n, 1))
    A_ub = np.vstack([np.hstack([A, -ones]), np.hstack([-A, -ones])])
    b_ub = np.concatenate([-base, base])
    c = np.zeros(deg + 1)
    c[-1] = 1.0
    r = linprog(c, A_ub=A_ub, b_ub=b_ub, bounds=[(None, None)] * (deg + 1), method="highs")
    coef = r.x[:deg].astype(np.float32)
    p = 1.0 + sum(float(coef[k]) * f ** (k + 1) for k in range(deg))
    return coef, float(np.abs(p / t - 1.0).max())


if __name__ == "__main__":
    coef, err = fit()
    for i, c in enumerate(coef, 1):
        print(f"kExp2C{i} = {float(c).hex()}  ({float(c):.9g})")
    print(f"max relative error on [-1/2, 1/2]: {err:.3e}")
