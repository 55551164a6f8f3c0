"""bench.py on the CPU: roofline.traffic comes from counter records committed under
profiles/ and must be reported only while the measured kernel's sources are unchanged; a
run asked for more than one GPU is refused."""

import json
import os
import shutil

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def records():
    out = []
    for name in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if name.endswith(".md"):
            with open(os.path.join(ROOT, "profiles", name)) as f:
                out += [json.loads(l[len("record: "):]) for l in f if l.startswith("record: ")]
    return out


def test_records_are_well_formed():
    recs = records()
    assert recs, "no traffic record under profiles/"
    for r in recs:
        assert r["bytes_per_launch"] == r["fetch_bytes"] + r["write_bytes"] or \
            abs(r["bytes_per_launch"] - r["fetch_bytes"] - r["write_bytes"]) <= 1
        assert 0.5 < r["fetch_factor"] < 4 and 0.5 < r["write_factor"] < 4
        assert len(r["source_sha256"]) == 64


@pytest.mark.parametrize("kernel,workload,src", [("bwd_main_kernel", "gqa_fwd_bwd", "attn_bwd.hip"),
                                                 ("fwd_kernel", "long_context_fwd", "attn_fwd.hip")])
def test_traffic_goes_null_when_the_kernel_changes(tmp_path, monkeypatch, kernel, workload, src):
    root = tmp_path / "repo"
    shutil.copytree(os.path.join(ROOT, "profiles"), root / "profiles")
    shutil.copytree(os.path.join(ROOT, "exact_attention_27_amd", "csrc"), root / "exact_attention_27_amd" / "csrc")
    monkeypatch.setattr(bench, "ROOT", str(root))
    rec = [r for r in records() if r["kernel"] == kernel and r["workload"] == workload]
    got = bench.traffic_record(kernel, workload)
    if rec and got is None:
        pytest.skip("record taken for other sources than these (counters not retaken yet)")
    if rec:
        assert got == rec[0]["bytes_per_launch"]
    path = root / "exact_attention_27_amd" / "csrc" / src
    path.write_bytes(path.read_bytes() + b"\n// changed\n")
    assert bench.traffic_record(kernel, workload) is None
    assert bench.traffic_record(kernel, "no_such_workload") is None


def test_mfma_ceiling_probe_is_optional_without_a_gpu():
    """bench.py runs the stand-alone MFMA ceiling probe as a child process; without a GPU
    (or without the built probe) it reports null instead of failing."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the probe would run")
    assert bench.mfma_ceiling() is None


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    """One GPU is the scope: --gpus above 1 exits with status 2 and says so, before any GPU
    work (this runs without one)."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in (r.stdout + r.stderr)
    assert '"metric"' not in r.stdout
