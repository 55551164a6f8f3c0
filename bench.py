"""Benchmark: exact attention forward + backward on one MI355X.

One step is one pass of the whole path over one batch of seeded synthetic inputs
already resident in device memory: attn_fwd (O, LSE) then the three backward launches
(preprocess, dK/dV main kernel, dQ kernel) giving dQ, dK, dV.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints one JSON line.  value = algorithmic TFLOP/s of the step, where a step's flop
count is fwd + bwd with fwd = 4*B*Hq*S^2*d (halved when causal) and bwd = 2.5 * fwd.
The roofline object is for the dominant kernel (the backward dK/dV kernel, timed with
HIP events on the stream it runs on, inside the timed region; its algorithmic flop is
the four products it performs, 2.0x the forward's).  cpu_baseline is the
fp64 oracle timed on this host on a bounded sample of the same workload.
"""

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd bf16 TFLOPS and % of MI355X MFMA peak, S=2k–32k, d=128"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, published (256 CU x 4096 flop/clk x 2.4 GHz)
VARIANT_NAMES = {0: "auto", 1: "pingpong", 2: "fourwave"}



def workload_names():
    import workloads
    names = {w.name: n for n, w in workloads.WORKLOADS.items()}
    names.update({w.name: n for n, w in workloads.VARLEN_WORKLOADS.items()})
    return names


def get_workload(name):
    import workloads
    n = workload_names()[name]
    return workloads.WORKLOADS[n] if n in workloads.WORKLOADS else workloads.VARLEN_WORKLOADS[n]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa_fwd_bwd", choices=sorted(workload_names()))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    ap.add_argument("--exp-mode", type=int, default=None)
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--variant", type=int, default=None,
                    help="forward schedule: 0 auto (default), 1 ping-pong, 2 four-wave")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run a plain device copy of MIB MiB (3 times): the "
                         "reference kernel that scales rocprofv3 FETCH_SIZE/WRITE_SIZE into bytes")
    return ap.parse_args()


def traffic_record(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the counter record committed under
    profiles/ (rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled by the same counter's reading
    for a plain device copy), or None when there is no record or the kernel's sources have
    changed since it was taken (the record holds their SHA-256)."""
    h = hashlib.sha256()
    for n in ("attn_bwd.hip", "attn_device.h", "attn_kernels.h") if kernel.startswith("bwd") else \
             ("attn_fwd.hip", "attn_device.h", "attn_kernels.h"):
        with open(os.path.join(ROOT, "exact_attention_27_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("record: "):
                    continue
                rec = json.loads(line[len("record: "):])
                if rec.get("kernel") == kernel and rec.get("workload") == workload and \
                        rec.get("source_sha256") == h.hexdigest():
                    return int(rec["bytes_per_launch"])
    return None


def copy_calibration(mib: int) -> None:
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "calls": 3}), flush=True)


def mfma_ceiling():
    """The chip's sustained dense bf16 MFMA rate with N(0,1) bf16 operands, from the
    stand-alone probe (exact_attention_27_amd/csrc/probes/mfma_ceiling.hip, built by
    build()), run as a child process; None if the probe is not built or fails."""
    exe = os.path.join(ROOT, "exact_attention_27_amd", "probes", "mfma_ceiling")
    if not os.path.exists(exe):
        return None
    import subprocess
    try:
        r = subprocess.run([exe, "--json"], capture_output=True, text=True, timeout=120)
        rec = json.loads(r.stdout.strip().splitlines()[-1]) if r.returncode == 0 else None
    except (subprocess.SubprocessError, ValueError, IndexError):
        rec = None
    if rec is None:
        return None
    return {"value": rec["tflops"], "unit": "TFLOP/s", "operands": "random N(0,1) bf16",
            "probe": "csrc/probes/mfma_ceiling.hip, 8 launches of back-to-back v_mfma_f32_32x32x16_bf16, "
                     "2 waves per SIMD, after the timed region"}


def blas_threads():
    """(threads, library) of the BLAS numpy uses on this host, as threadpoolctl reports them."""
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            return max(i.get("num_threads", 1) for i in info), \
                "/".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info}))
    except Exception:  # noqa: BLE001
        pass
    return os.cpu_count() or 1, "unknown"


def cpu_baseline(w, inputs, target_s):
    """The fp64 oracle (fwd + bwd of one (batch, query head) pair at a time, at the
    workload's full S) on this host, until about target_s seconds have passed."""
    import numpy as np
    import oracle
    threads, blas = blas_threads()
    x = {n: inputs[n] for n in ("q", "k", "v", "do")}
    heads, flop, t0 = 0, 0.0, time.perf_counter()
    per_head_fwd = w.fwd_flop() / (w.B * w.Hq)
    do_bwd = "bwd" in w.passes
    for b in range(w.B):
        for h in range(w.Hq):
            hk = oracle.kv_head_of(h, w.Hq, w.Hkv)
            q = x["q"][b, h].float().numpy().astype(np.float64)
            k = x["k"][b, hk].float().numpy().astype(np.float64)
            v = x["v"][b, hk].float().numpy().astype(np.float64)
            oracle.head_forward(q, k, v, w.scale, w.causal)
            flop += per_head_fwd
            if do_bwd:
                do = x["do"][b, h].float().numpy().astype(np.float64)
                oracle.head_backward(q, k, v, do, w.scale, w.causal)
                flop += 2.5 * per_head_fwd
            heads += 1
            if time.perf_counter() - t0 >= target_s:
                break
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "blas": blas, "kind": "oracle",
        "sample": f"fp64 numpy oracle, {'fwd+bwd' if do_bwd else 'fwd'} of {heads} of {w.B * w.Hq} "
                  f"(batch, query head) pairs at full S={w.S}, d={w.d}, {dt:.1f} s; algorithmic flop",
    }


def cpu_baseline_varlen(w, inputs, target_s):
    """The fp64 oracle forward of one (sequence, query head) pair at a time, sequences in
    packed order, until about target_s seconds have passed."""
    import numpy as np
    import oracle
    threads, blas = blas_threads()
    cu = inputs["cu_seqlens"].tolist()
    pairs, toks, flop, t0 = 0, 0, 0.0, time.perf_counter()
    done = False
    for s in range(len(cu) - 1):
        a, n = cu[s], cu[s + 1] - cu[s]
        for h in range(w.Hq):
            hk = oracle.kv_head_of(h, w.Hq, w.Hkv)
            f = lambda x, hh: x[a:a + n, hh].float().numpy().astype(np.float64)
            oracle.head_forward(f(inputs["q"], h), f(inputs["k"], hk), f(inputs["v"], hk), w.scale, w.causal)
            flop += 4.0 * n * n * w.d / (2 if w.causal else 1)
            pairs += 1
            toks += n
            if time.perf_counter() - t0 >= target_s:
                done = True
                break
        if done:
            break
    dt = time.perf_counter() - t0
    return {
        "value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "blas": blas, "kind": "oracle",
        "sample": f"fp64 numpy oracle, fwd of {pairs} of {w.n * w.Hq} (sequence, query head) pairs "
                  f"({toks} query rows) of the packed batch, d={w.d}, {dt:.1f} s; algorithmic flop",
    }


def main_varlen(args, w):
    """Time the packed forward (attn_fwd_varlen) on a variable-length workload."""
    import torch
    import exact_attention_27_amd as ea
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    host = workloads.make_varlen_inputs(w)
    t = {n: x.to(dev) for n, x in host.items()}
    lens = w.lengths()
    total = sum(lens)
    opt = ea.attn_default_options()
    if args.exp_mode is not None:
        opt.exp_mode = args.exp_mode
    if args.tau is not None:
        opt.tau = args.tau
    if args.variant is not None:
        opt.variant = args.variant
    o = torch.empty_like(t["q"])
    lse = torch.empty((w.Hq, total), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        ea.attn_fwd_varlen(t["q"], t["k"], t["v"], t["cu_seqlens"], max(lens), w.scale, w.causal, o=o, lse=lse,
                           opt=opt, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for _ in range(args.steps):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    fwd_ms = ev[0].elapsed_time(ev[1]) / args.steps
    flop = w.fwd_flop()
    value = flop / (ms_step * 1e-3) / 1e12
    fwd_tf = flop / (fwd_ms * 1e-3) / 1e12
    roofline = {"kernel": "fwd_kernel", "bound": "mfma", "achieved": round(fwd_tf, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_record("fwd_kernel", w.name),
                "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "avg_launch_ms": round(fwd_ms, 4)}
    ceiling = mfma_ceiling()
    if ceiling:
        roofline["frac_of_measured_ceiling"] = round(fwd_tf / ceiling["value"], 4)
    cpu = None if args.no_cpu_baseline else cpu_baseline_varlen(w, host, args.cpu_seconds)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "sequences": w.n, "lengths": f"{min(lens)}..{max(lens)} log-uniform",
                   "total_tokens": total, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "causal": w.causal,
                   "passes": "fwd", "exp_mode": int(opt.exp_mode), "tau": float(opt.tau),
                   "variant": VARIANT_NAMES.get(int(opt.variant), int(opt.variant)), "step_flop": flop},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline, "mfma_ceiling": ceiling, "breakdown": {"fwd_ms": round(fwd_ms, 4), "fwd_tflops": round(fwd_tf, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path (attention "
              "would shard over batch and heads with no exchange, each GPU running these kernels "
              "on its share); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_27_amd as ea
    import workloads

    w = get_workload(args.workload)
    if isinstance(w, workloads.VarlenWorkload):
        main_varlen(args, w)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    host = workloads.make_inputs(w)
    t = {n: x.to(dev) for n, x in host.items()}
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    opt = ea.attn_default_options()
    if args.exp_mode is not None:
        opt.exp_mode = args.exp_mode
    if args.tau is not None:
        opt.tau = args.tau
    if args.variant is not None:
        opt.variant = args.variant
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(1, ea.attn_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.S, w.d)), dtype=torch.uint8, device=dev)
    do_bwd = "bwd" in w.passes
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        ea.attn_fwd_ex(q, k, v, w.scale, w.causal, o, lse, opt=opt, stream=stream)
        if ev:
            ev[1].record(stream)
        if do_bwd:
            for ph, e in ((ea.ATTN_BWD_PREPROCESS, 2), (ea.ATTN_BWD_MAIN, 3), (ea.ATTN_BWD_DQ, 4)):
                ea.attn_bwd_phase(ph, q, k, v, o, lse, do, w.scale, w.causal, dq, dk, dv, ws, opt=opt, stream=stream)
                if ev:
                    ev[e].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # A forward-only step is one launch: one event pair around the whole timed loop gives
    # its average duration back to back.  The backward's phases need events between them.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps if do_bwd else 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if do_bwd:
        for i in range(args.steps):
            step(evs[i])
    else:
        evs[0][0].record(stream)
        for i in range(args.steps):
            step()
        evs[0][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms_step = elapsed * 1e3 / args.steps
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    phase_ms = {}
    if do_bwd:
        phase_ms["bwd_pre"] = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
        phase_ms["bwd_main"] = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
        phase_ms["bwd_dq"] = sum(e[3].elapsed_time(e[4]) for e in evs) / args.steps
    fwd_tf = w.fwd_flop() / (fwd_ms * 1e-3) / 1e12
    flop = w.fwd_flop() + (w.bwd_flop() if do_bwd else 0.0)
    value = flop / (ms_step * 1e-3) / 1e12

    if do_bwd:
        # The dK/dV kernel performs four of the backward's five counted products (S, dP,
        # dV, dK): 2.0x the forward's flop; the dQ kernel does the fifth (plus recomputing S
        # and dP, which the flop convention does not count).
        main_ms = phase_ms["bwd_main"]
        achieved = 2.0 * w.fwd_flop() / (main_ms * 1e-3) / 1e12
        dominant = "bwd_main_kernel"
    else:
        main_ms = fwd_ms
        achieved = fwd_tf
        dominant = "fwd_kernel"
    traffic = traffic_record(dominant, w.name)
    roofline = {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "avg_launch_ms": round(main_ms, 4)}
    breakdown = {"fwd_ms": round(fwd_ms, 4), "fwd_tflops": round(fwd_tf, 2),
                 "fwd_frac_of_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4)}
    if do_bwd:
        bwd_ms = sum(phase_ms.values())
        bwd_tf = w.bwd_flop() / (bwd_ms * 1e-3) / 1e12
        breakdown.update({k + "_ms": round(v, 4) for k, v in phase_ms.items()})
        breakdown.update({"bwd_ms": round(bwd_ms, 4), "bwd_tflops": round(bwd_tf, 2),
                          "bwd_frac_of_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4)})

    ceiling = mfma_ceiling()
    if ceiling:
        roofline["frac_of_measured_ceiling"] = round(achieved / ceiling["value"], 4)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, host, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "S": w.S, "d": w.d,
                   "causal": w.causal, "passes": "+".join(w.passes), "exp_mode": int(opt.exp_mode),
                   "tau": float(opt.tau), "variant": VARIANT_NAMES.get(int(opt.variant), int(opt.variant)), "step_flop": flop},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline, "mfma_ceiling": ceiling, "breakdown": breakdown, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
