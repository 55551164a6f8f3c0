"""Checks on the gfx950 assembly of the kernels (compiled here, no GPU needed):

* m0 is written only by the LDS-DMA sequences (s_mov_b32 m0 right before a
  global_load_lds): the compiler itself uses m0 nowhere, which is what makes the inline
  asm's m0 clobber safe;
* no packed-fp32 VALU instructions (v_pk_add/mul/fma_f32), which the build disables;
* nothing is written through the scalar data cache (no s_store / s_buffer_store /
  scalar atomics);
* no kernel uses scratch (register spills).
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_27_amd", "csrc")
HIPCC = os.environ.get("HIPCC") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc"))

pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa")
    procs = {}
    for name in ("attn_fwd", "attn_bwd"):
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-Wno-inline-asm", "-I", CSRC, "-I", os.path.join(ROOT, "include"), "-S",
               "--cuda-device-only", "-o", str(out / f"{name}.s"), os.path.join(CSRC, f"{name}.hip")]
        procs[name] = subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, text=True)
    texts = {}
    for name, p in procs.items():
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, err[-2000:]
        texts[name] = (out / f"{name}.s").read_text()
    return texts


def instructions(text):
    for line in text.splitlines():
        s = line.strip()
        if not s or s.startswith((";", ".", "//")) or s.endswith(":"):
            continue
        yield s.split(";")[0].strip()


def test_m0_written_only_by_the_lds_dma(isa):
    for name, text in isa.items():
        ins = list(instructions(text))
        for i, s in enumerate(ins):
            if re.search(r"\bm0\b", s):
                assert s.startswith("s_mov_b32 m0,"), f"{name}: compiler use of m0: {s}"
                nxt = [t for t in ins[i + 1:i + 3] if not t.startswith("s_nop")]
                assert nxt and nxt[0].startswith("global_load_lds"), f"{name}: m0 write not followed by the DMA: {s}"


def test_no_packed_fp32_and_no_scalar_stores(isa):
    for name, text in isa.items():
        for s in instructions(text):
            assert not re.match(r"v_pk_(add|mul|fma)_f32", s), f"{name}: packed fp32: {s}"
            assert not re.match(r"s_(buffer_)?(store|atomic)", s), f"{name}: scalar store: {s}"
            assert not s.startswith(("s_dcache_wb", "s_dcache_discard")), f"{name}: {s}"


def test_no_scratch(isa):
    scratch = {}
    for text in isa.values():
        # kernel metadata: ".name: <symbol>" followed by ".private_segment_fixed_size: <bytes>"
        for m in re.finditer(r"\.name:\s+(\S+)\n\s+\.private_segment_fixed_size:\s+(\d+)", text):
            scratch[m.group(1)] = int(m.group(2))
    assert len([k for k in scratch if "fwd_kernel" in k]) == 32, sorted(scratch)  # 2 d x 2 causal x 2 exp x 2 layouts x 2 schedules
    # preprocess 2 d; dQ 2 d x 2 causal x 2 exp; dK/dV: d = 64 four-wave (x 2 causal x 2 exp), d = 128 eight-wave
    # (x 2 causal x 2 exp) and four-wave (x 2 causal, hardware exponential only); each dense and packed
    assert len([k for k in scratch if "bwd_" in k]) == 40, sorted(scratch)
    for kernel, n in scratch.items():
        assert n == 0, f"{kernel} uses {n} bytes of scratch"
