"""Benchmark: exact attention forward + backward on one MI355X.

One step is one pass of the whole path over one batch of seeded synthetic inputs
already resident in device memory: attn_fwd (O, LSE) then the backward's three launches
(preprocess, dQ kernel, dK/dV kernel) giving dQ, dK, dV.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-configs]

Prints one JSON line.  value = algorithmic TFLOP/s of the step, where a step's flop
count is fwd + bwd with fwd = 4*B*Hq*S^2*d (halved when causal) and bwd = 2.5 * fwd.
The roofline object is for the dominant kernel (the backward's dK/dV kernel, timed with
HIP events on the stream it runs on, inside the timed region; its algorithmic flop is
the four products it performs, 2.0x the forward's).  "configs" adds, after the timed
region, median and minimum per-launch times of the other headline configurations (the
2k prefill forward, the 32k long-context forward and the 4k backward), each timed over
groups of back-to-back calls with one event pair per group (an event pair around every
call would add the events' own cost to each 0.08 ms prefill launch), and of this
workload's own passes (from the timed steps' per-launch events).  "clock" is the shader clock and board
power (amdsmi) while the same step repeats for a few seconds right after the timed region
(amdsmi refreshes about once a second, slower than the timed region lasts); the 32k
forward's entry has one too.  cpu_baseline is the fp64 oracle timed on this host on a
bounded sample of the same workload.
"""

import argparse
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import threading
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
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration timings that follow the timed region")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    ap.add_argument("--exp-mode", type=int, default=None)
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--variant", type=int, default=None,
                    help="forward schedule: 0 auto (default), 1 ping-pong, 2 four-wave")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark, print one JSON line per sequence length S = 2k..32k "
                         "(H=16, d=128, causal, B*S = 32768 tokens): forward and backward per-call times "
                         "over groups of back-to-back calls")
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
            if "bwd" in w.passes:
                oracle.head_backward(f(inputs["q"], h), f(inputs["k"], hk), f(inputs["v"], hk), f(inputs["do"], h),
                                     w.scale, w.causal)
                flop += 2.5 * 4.0 * n * n * w.d / (2 if w.causal else 1)
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
        "sample": f"fp64 numpy oracle, {'+'.join(w.passes)} of {pairs} of {w.n * w.Hq} (sequence, query head) pairs "
                  f"({toks} query rows) of the packed batch, d={w.d}, {dt:.1f} s; algorithmic flop",
    }


class VarlenRun:
    """A packed workload's tensors on the GPU and its passes: attn_fwd_varlen and, for
    backward workloads, attn_bwd_varlen (workspace allocated once, outside any timing)."""

    def __init__(self, w, opt):
        import torch
        import exact_attention_27_amd as ea
        import workloads
        self.torch, self.ea, self.w, self.opt = torch, ea, w, opt
        self.with_bwd = "bwd" in w.passes
        dev = torch.device("cuda:0")
        host = workloads.make_varlen_inputs(w, with_do=self.with_bwd)
        self.host = host
        self.t = {n: x.to(dev) for n, x in host.items()}
        self.lens = w.lengths()
        self.total = sum(self.lens)
        self.ms = max(self.lens)
        self.o = torch.empty_like(self.t["q"])
        self.lse = torch.empty((w.Hq, self.total), dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream()
        if self.with_bwd:
            self.dq = torch.empty_like(self.t["q"])
            self.dk = torch.empty_like(self.t["k"])
            self.dv = torch.empty_like(self.t["v"])
            nb = ea.attn_bwd_varlen_workspace_bytes(w.n, self.total, w.Hq, w.Hkv, w.d)
            self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)

    def fwd(self):
        t, w = self.t, self.w
        self.ea.attn_fwd_varlen(t["q"], t["k"], t["v"], t["cu_seqlens"], self.ms, w.scale, w.causal, o=self.o,
                                lse=self.lse, opt=self.opt, stream=self.stream)

    def bwd(self):
        t, w = self.t, self.w
        self.ea.attn_bwd_varlen(t["q"], t["k"], t["v"], self.o, self.lse, t["do"], t["cu_seqlens"], self.ms, w.scale,
                                w.causal, dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws, opt=self.opt,
                                stream=self.stream)

    def grouped(self, reps, target_ms=2.0):
        """Per-call times of each pass over groups of back-to-back calls (as DenseRun.grouped)."""
        torch, s = self.torch, self.stream
        out = {}
        self.fwd()
        for name, fn in (("fwd", self.fwd),) + ((("bwd", self.bwd),) if self.with_bwd else ()):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn()
            e1.record(s)
            torch.cuda.synchronize()
            g = max(1, min(200, int(target_ms / max(e0.elapsed_time(e1), 1e-3))))
            ms = []
            for _ in range(reps):
                e0.record(s)
                for _ in range(g):
                    fn()
                e1.record(s)
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1) / g)
            out[name] = ms
        return out


def varlen_config_entry(w, opt, reps):
    """Per-call statistics of a packed workload's passes (after the timed region)."""
    run = VarlenRun(w, opt)
    gr = run.grouped(reps)
    out = {"shape": {"sequences": w.n, "lengths": f"{min(run.lens)}..{max(run.lens)}", "total_tokens": run.total,
                     "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "causal": w.causal},
           "groups": reps, "timing": "per call, over groups of back-to-back calls of about 2 ms",
           "fwd": pass_stats(gr["fwd"], w.fwd_flop())}
    if run.with_bwd:
        out["bwd"] = pass_stats(gr["bwd"], w.bwd_flop())
    del run
    return out


def main_varlen(args, w):
    """Time a packed workload: attn_fwd_varlen, and attn_bwd_varlen for backward workloads."""
    import torch
    import exact_attention_27_amd as ea
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lens = w.lengths()
    total = sum(lens)
    opt = ea.attn_default_options()
    if args.exp_mode is not None:
        opt.exp_mode = args.exp_mode
    if args.tau is not None:
        opt.tau = args.tau
    if args.variant is not None:
        opt.variant = args.variant
    run = VarlenRun(w, opt)
    host = run.host
    stream = run.stream

    def step(ev=None):
        run.fwd()
        if ev:
            ev[1].record(stream)
        if run.with_bwd:
            run.bwd()
            if ev:
                ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    fwd_ms = statistics.mean(e[0].elapsed_time(e[1]) for e in evs)
    bwd_ms = statistics.mean(e[1].elapsed_time(e[2]) for e in evs) if run.with_bwd else None
    flop = w.fwd_flop() + (w.bwd_flop() if run.with_bwd else 0.0)
    value = flop / (ms_step * 1e-3) / 1e12
    fwd_tf = w.fwd_flop() / (fwd_ms * 1e-3) / 1e12
    roofline = {"kernel": "fwd_kernel", "bound": "mfma", "achieved": round(fwd_tf, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_record("fwd_kernel", w.name),
                "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "avg_launch_ms": round(fwd_ms, 4)}
    if run.with_bwd:
        # The backward dominates a training step; its three launches run inside one call
        # (attn_bwd_varlen), timed as one: algorithmic backward flop over the call's time.
        bwd_tf = w.bwd_flop() / (bwd_ms * 1e-3) / 1e12
        roofline = {"kernel": "attn_bwd_varlen (preprocess, dQ and dK/dV launches)", "bound": "mfma",
                    "achieved": round(bwd_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(bwd_tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                    "traffic_unit": "bytes per launch (no counter record for the packed backward)",
                    "avg_launch_ms": round(bwd_ms, 4)}
    ceiling = mfma_ceiling()
    if ceiling:
        roofline["frac_of_measured_ceiling"] = round(roofline["achieved"] / ceiling["value"], 4)
    cpu = None if args.no_cpu_baseline else cpu_baseline_varlen(w, host, args.cpu_seconds)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "sequences": w.n, "lengths": f"{min(lens)}..{max(lens)} log-uniform",
                   "total_tokens": total, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "causal": w.causal,
                   "passes": "+".join(w.passes), "exp_mode": int(opt.exp_mode), "tau": float(opt.tau),
                   "variant": VARIANT_NAMES.get(int(opt.variant), int(opt.variant)), "step_flop": flop},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline, "mfma_ceiling": ceiling,
        "breakdown": {"fwd_ms": round(fwd_ms, 4), "fwd_tflops": round(fwd_tf, 2),
                      **({"bwd_ms": round(bwd_ms, 4), "bwd_tflops": round(w.bwd_flop() / (bwd_ms * 1e-3) / 1e12, 2)}
                         if run.with_bwd else {})},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


class ClockSampler:
    """Samples the shader clock (mean over the XCDs) and board power with amdsmi in a
    background thread.  The values amdsmi reports are refreshed about once a second, so
    they describe a load only after it has run for over a second; stats() drops the
    first `settle_s` seconds of samples.  None where amdsmi is absent."""

    def __init__(self, period_s=0.02, settle_s=1.2):
        self.period, self.settle = period_s, settle_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception:  # noqa: BLE001
            self._smi = None

    def _run(self):
        t0 = time.perf_counter()
        while not self._stop.is_set():
            try:
                m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
                c = [x for x in m.get("current_gfxclks", []) if isinstance(x, (int, float)) and 0 < x < 10000]
                p = m.get("current_socket_power")
                if c:
                    self.samples.append((time.perf_counter() - t0, sum(c) / len(c),
                                         p if isinstance(p, (int, float)) else None))
            except Exception:  # noqa: BLE001
                return
            time.sleep(self.period)

    def __enter__(self):
        if self._smi is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join(timeout=5)
        return False

    def stats(self):
        s = [x for x in self.samples if x[0] >= self.settle]
        if not s:
            return None
        clk = [x[1] for x in s]
        pwr = [x[2] for x in s if x[2] is not None]
        out = {"sclk_mhz_mean": round(statistics.mean(clk), 1), "sclk_mhz_min": round(min(clk), 1),
               "sclk_mhz_max": round(max(clk), 1), "samples": len(s)}
        if pwr:
            out["power_w_mean"] = round(statistics.mean(pwr), 1)
        return out


def sustained_clock(run, seconds=2.6):
    """The shader clock and board power while `run`'s step repeats back to back for about
    `seconds` (amdsmi refreshes its readings about once a second, too slowly for the short
    timed region itself): the clock the timed steps run at, measured right after them."""
    sampler = ClockSampler()
    if sampler._smi is None:
        return None
    with sampler:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(8):
                run.step()
            run.torch.cuda.synchronize()
    st = sampler.stats()
    if st:
        st["source"] = (f"amdsmi current_gfxclks (mean of the XCDs) and current_socket_power, sampled while "
                        f"the same step repeated for {seconds:.1f} s after the timed region; first "
                        f"{sampler.settle:.1f} s dropped (amdsmi refreshes about once a second)")
    return st


def pass_stats(ms_list, flop):
    """Median / min / mean per-launch time of one pass and its algorithmic rate."""
    med, mn = statistics.median(ms_list), min(ms_list)
    return {"ms_median": round(med, 4), "ms_min": round(mn, 4), "ms_mean": round(statistics.mean(ms_list), 4),
            "tflops_median": round(flop / (med * 1e-3) / 1e12, 2), "tflops_best": round(flop / (mn * 1e-3) / 1e12, 2),
            "frac_of_peak_median": round(flop / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


class DenseRun:
    """Device-resident inputs and outputs of a dense workload, and one step of the path with
    an event after each launch (forward, then the backward's phases in their order)."""

    PHASES = (("bwd_pre", "ATTN_BWD_PREPROCESS"), ("bwd_dq", "ATTN_BWD_DQ"), ("bwd_main", "ATTN_BWD_MAIN"))

    def __init__(self, w, opt, with_bwd):
        import torch
        import exact_attention_27_amd as ea
        import workloads
        self.torch, self.ea, self.w, self.opt, self.with_bwd = torch, ea, w, opt, with_bwd
        self.host = workloads.make_inputs(w)
        t = {n: x.to("cuda:0") for n, x in self.host.items()}
        self.q, self.k, self.v, self.do = t["q"], t["k"], t["v"], t["do"]
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device="cuda:0")
        self.dq, self.dk, self.dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        nb = ea.attn_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.S, w.d)
        self.ws = torch.empty(max(1, nb), dtype=torch.uint8, device="cuda:0")
        self.stream = torch.cuda.current_stream()
        self.names = ["fwd"] + ([n for n, _ in self.PHASES] if with_bwd else [])

    def step(self, ev=None):
        ea, w, s = self.ea, self.w, self.stream
        if ev:
            ev[0].record(s)
        ea.attn_fwd_ex(self.q, self.k, self.v, w.scale, w.causal, self.o, self.lse, opt=self.opt, stream=s)
        if ev:
            ev[1].record(s)
        if self.with_bwd:
            for i, (_, ph) in enumerate(self.PHASES):
                ea.attn_bwd_phase(getattr(ea, ph), self.q, self.k, self.v, self.o, self.lse, self.do, w.scale,
                                  w.causal, self.dq, self.dk, self.dv, self.ws, opt=self.opt, stream=s)
                if ev:
                    ev[2 + i].record(s)

    def timed(self, steps, warmup):
        """Runs warmup untimed steps, then `steps` steps with events; returns (wall seconds of
        the timed steps, {launch name: [ms per step]})."""
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(self.names) + 1)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(evs[i])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        ms = {n: [e[j].elapsed_time(e[j + 1]) for e in evs] for j, n in enumerate(self.names)}
        return elapsed, ms

    def grouped(self, reps, target_ms=2.0):
        """Per-launch times of the forward, and of the whole backward, over groups of
        back-to-back calls: one event pair around each group of g calls (g chosen so that a
        group lasts about target_ms), `reps` groups.  An event pair around every single call
        adds the events' own cost to each launch (several microseconds, which a 0.08 ms
        launch feels); grouped calls measure what a stream of calls sustains.  Returns
        {"fwd": [ms per call], "bwd": [ms per call]} (bwd only for backward workloads)."""
        torch, ea, w, s = self.torch, self.ea, self.w, self.stream

        def fwd():
            ea.attn_fwd_ex(self.q, self.k, self.v, w.scale, w.causal, self.o, self.lse, opt=self.opt, stream=s)

        def bwd():
            for _, ph in self.PHASES:
                ea.attn_bwd_phase(getattr(ea, ph), self.q, self.k, self.v, self.o, self.lse, self.do, w.scale,
                                  w.causal, self.dq, self.dk, self.dv, self.ws, opt=self.opt, stream=s)

        out = {}
        for name, fn in (("fwd", fwd),) + ((("bwd", bwd),) if self.with_bwd else ()):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn()
            e1.record(s)
            torch.cuda.synchronize()
            g = max(1, min(200, int(target_ms / max(e0.elapsed_time(e1), 1e-3))))
            ms = []
            for _ in range(reps):
                e0.record(s)
                for _ in range(g):
                    fn()
                e1.record(s)
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1) / g)
            out[name] = ms
        return out


def config_entry(w, opt, steps, warmup, clock=False):
    """Per-launch statistics of one more dense workload (after the timed region): median and
    minimum over `steps` groups of back-to-back calls (DenseRun.grouped), and the backward's
    phases from an event pair around each launch."""
    with_bwd = "bwd" in w.passes
    run = DenseRun(w, opt, with_bwd)
    _, ms = run.timed(steps, warmup)
    gr = run.grouped(steps)
    out = {"shape": {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "S": w.S, "d": w.d, "causal": w.causal},
           "groups": steps, "timing": "per call, over groups of back-to-back calls of about 2 ms",
           "fwd": pass_stats(gr["fwd"], w.fwd_flop())}
    if with_bwd:
        out["bwd"] = pass_stats(gr["bwd"], w.bwd_flop())
        out["bwd"]["phases_ms_median"] = {n: round(statistics.median(ms[n]), 4) for n, _ in DenseRun.PHASES}
    if clock:
        out["clock"] = sustained_clock(run)
    del run
    return out


def sweep(opt):
    """Forward and backward rates against the sequence length at a fixed token count
    (B * S = 32768, H = 16, d = 128, causal, bf16 N(0,1) inputs seeded by S), one JSON line
    per length."""
    import torch
    import workloads
    for S in (2048, 4096, 8192, 16384, 32768):
        B = 32768 // S
        w = workloads.Workload(100 + S // 1024, f"sweep_S{S}", B, 16, 16, S, 128, True, ("fwd", "bwd"))
        run = DenseRun(w, opt, True)
        run.timed(3, 3)  # warm-up
        gr = run.grouped(10)
        print(json.dumps({"S": S, "B": B, "H": 16, "d": 128, "causal": True,
                          "fwd": pass_stats(gr["fwd"], w.fwd_flop()), "bwd": pass_stats(gr["bwd"], w.bwd_flop())}),
              flush=True)
        del run
        torch.cuda.empty_cache()


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

    if args.sweep:
        torch.cuda.set_device(torch.device("cuda:0"))
        sweep(ea.attn_default_options())
        return
    w = get_workload(args.workload)
    if isinstance(w, workloads.VarlenWorkload):
        main_varlen(args, w)
        return
    torch.cuda.set_device(torch.device("cuda:0"))
    opt = ea.attn_default_options()
    if args.exp_mode is not None:
        opt.exp_mode = args.exp_mode
    if args.tau is not None:
        opt.tau = args.tau
    if args.variant is not None:
        opt.variant = args.variant
    do_bwd = "bwd" in w.passes
    run = DenseRun(w, opt, do_bwd)
    host = run.host

    # The timed region: exactly args.steps steps, synchronized on both sides.
    elapsed, ms = run.timed(args.steps, args.warmup)
    clock = None if args.no_configs else sustained_clock(run)

    ms_step = elapsed * 1e3 / args.steps
    flop = w.fwd_flop() + (w.bwd_flop() if do_bwd else 0.0)
    value = flop / (ms_step * 1e-3) / 1e12
    step_ms = [sum(x) for x in zip(*ms.values())]  # event-timed launches of each step
    fwd_ms = statistics.mean(ms["fwd"])
    fwd_tf = w.fwd_flop() / (fwd_ms * 1e-3) / 1e12
    phase_ms = {n: statistics.mean(ms[n]) for n, _ in DenseRun.PHASES} if do_bwd else {}

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
    if clock:
        roofline["frac_at_measured_clock"] = round(achieved / (PEAK_BF16_TFLOPS * clock["sclk_mhz_mean"] / 2400.0), 4)
    breakdown = {"fwd_ms": round(fwd_ms, 4), "fwd_tflops": round(fwd_tf, 2),
                 "fwd_frac_of_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
                 "step_ms_median": round(statistics.median(step_ms), 4), "step_ms_min": round(min(step_ms), 4)}
    if do_bwd:
        bwd_ms = sum(phase_ms.values())
        bwd_tf = w.bwd_flop() / (bwd_ms * 1e-3) / 1e12
        breakdown.update({k + "_ms": round(v, 4) for k, v in phase_ms.items()})
        breakdown.update({"bwd_ms": round(bwd_ms, 4), "bwd_tflops": round(bwd_tf, 2),
                          "bwd_frac_of_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4)})
    del run

    # After the timed region: the other headline configurations, and this one's passes.
    configs = None
    if not args.no_configs:
        configs = {}
        own = {"fwd": pass_stats(ms["fwd"], w.fwd_flop())}
        if do_bwd:
            own["bwd"] = pass_stats([sum(x) for x in zip(*(ms[n] for n, _ in DenseRun.PHASES))], w.bwd_flop())
        configs[w.name] = own
        extra = {"prefill_fwd": (50, 10, False), "long_context_fwd": (20, 3, True), "bwd": (20, 5, False)}
        for name, (k, wu, clk) in extra.items():
            if name != w.name:
                configs[name] = config_entry(get_workload(name), opt, k, wu, clk)
                torch.cuda.empty_cache()
        configs["varlen_train_fwd_bwd"] = varlen_config_entry(get_workload("varlen_train_fwd_bwd"), opt, 10)
        torch.cuda.empty_cache()

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
                   "tau": float(opt.tau), "variant": VARIANT_NAMES.get(int(opt.variant), int(opt.variant)),
                   "step_flop": flop},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline, "clock": clock, "mfma_ceiling": ceiling, "breakdown": breakdown,
        "configs": configs, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
