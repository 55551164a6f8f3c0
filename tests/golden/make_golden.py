"""Write oracle_tiny.json: oracle outputs on one tiny seeded case (regression fixture).

Calls only the oracle and the seeded input generator.  Run from the repo root:
    python tests/golden/make_golden.py
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

CASE = dict(B=1, Hq=2, Hkv=1, S=7, d=4, seed=123, scale=0.5, causal=True)


def main():
    t = workloads.make_tensors(CASE["B"], CASE["Hq"], CASE["Hkv"], CASE["S"], CASE["d"], CASE["seed"])
    x = {n: t[n].float().numpy() for n in ("q", "k", "v", "do")}
    o, lse = oracle.attention_forward(x["q"], x["k"], x["v"], CASE["scale"], CASE["causal"])
    dq, dk, dv = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], CASE["scale"], CASE["causal"])
    out = {"case": CASE, "o": o.tolist(), "lse": lse.tolist(), "dq": dq.tolist(), "dk": dk.tolist(), "dv": dv.tolist()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
