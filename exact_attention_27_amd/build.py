"""Build libattn.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

Usage:  python -m exact_attention_27_amd.build     (or __graft_entry__.build())
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["attn_api.hip", "attn_fwd.hip", "attn_bwd.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libattn.so)")


def command(out: str = LIB):
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
        # Packed-fp32 VALU forms are kept out of every kernel.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-o", out,
    ] + [os.path.join(CSRC, s) for s in SOURCES]


PROBE_SRC = os.path.join(CSRC, "probes", "mfma_ceiling.hip")
PROBE_BIN = os.path.join(PKG, "probes", "mfma_ceiling")
# Further stand-alone probes: (source, binary).
PROBES = [
    (PROBE_SRC, PROBE_BIN),
    (os.path.join(CSRC, "probes", "dq_atomics.hip"), os.path.join(PKG, "probes", "dq_atomics")),
]


def build_probe(verbose: bool = True) -> str:
    """Compile the stand-alone probes (not part of the library: the MFMA ceiling and the
    fused-dQ atomic traffic) next to the package, as a check that they build; run them on
    a GPU to measure.  Returns the MFMA ceiling probe's path."""
    os.makedirs(os.path.dirname(PROBE_BIN), exist_ok=True)
    for src, out in PROBES:
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", out, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr}")
    return PROBE_BIN


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    build_probe()
