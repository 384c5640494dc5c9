"""Benchmark one Muon / MONA optimizer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A "step" is one full optimizer step over every matrix of the workload (MONA,
momentum, normalisation, Newton-Schulz, decoupled update), with gradients and
state already resident in HBM.  Rank 0 prints one JSON line with the step time
(the headline value), the dominant kernel's roofline (kernel durations
measured with HIP events on the launch stream), and the fp64 CPU oracle timed
on this host's cores on a bounded sample.
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Muon step ms per model + NS TFLOP/s (% MFMA peak), elementwise GB/s"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # MI355X dense MFMA
PEAK_HBM_GBPS = 8000.0
SCLK_NOMINAL_MHZ = 2400.0   # shader clock of the MFMA peak figures


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gram_tall_32x4096x16384")
    ap.add_argument("--variant", default=None, help="direct | gram (default: the workload's first)")
    ap.add_argument("--no-graph", action="store_true", help="launch kernels directly instead of a HIP graph")
    ap.add_argument("--mona-lite", action="store_true",
                    help="MONA workloads keep one bfloat16 MONA-Lite state instead of A and G_prev")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trace-steps", type=int, default=None, help="steps timed per launch (default: --steps)")
    ap.add_argument("--adamw", type=int, default=0, metavar="MELEMS",
                    help="only time muon_adamw_step over a synthetic set of MELEMS million vector-parameter "
                         "elements (bf16 grads) and print its own JSON line")
    ap.add_argument("--grad-kind", default=None, choices=("gaussian", "spectral", "spike", "expert"),
                    help="replace the workload's gradient recipe (counter runs: the profiler's counter mode "
                         "faults inside the QR the spectral and spike recipes call; the product launches "
                         "do not depend on the values)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB --steps times (counter calibration)")
    return ap.parse_args()


def kernel_source_hash():
    """sha256 of the NS product kernels' code and of the host code that
    configures their launches (ns_gemm.hip, the argument blocks in
    muon_kernels.h, muon_host.cpp; comments and whitespace removed):
    HBM-traffic figures in profiles/ apply only to the code they were
    measured on, and an edit of a comment does not change that code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in ("ns_gemm.hip", "muon_kernels.h", "muon_host.cpp"):
        path = os.path.join(ROOT, "newton_schulz_matrix_momentum_amd", "csrc", name)
        with open(path) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per NS GEMM launch measured with rocprofv3 FETCH_SIZE and
    WRITE_SIZE (scaled by a plain copy's readings), from
    profiles/<workload>_ns_gemm_traffic.md, or None when that file is absent
    or was measured on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "%s_ns_gemm_traffic.md" % workload)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_code_sha256") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe(args):
    import torch
    n = args.copy_probe << 20
    x = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": args.steps}), flush=True)


def adamw_probe(args):
    """AdamW over a synthetic vector-parameter set: 96 tensors whose sizes span
    three decades (norm weights to embedding rows), ``args.adamw`` million
    elements in all, bf16 gradients.  Kernel time from HIP events around the
    library's launches (muon_trace, grouped)."""
    import torch
    import newton_schulz_matrix_momentum_amd as nsm
    from newton_schulz_matrix_momentum_amd import _lib
    gen = torch.Generator().manual_seed(7)
    w = 10.0 ** (3.0 * torch.rand(96, generator=gen, dtype=torch.float64))
    sizes = [max(1, int(v)) for v in (w / w.sum() * args.adamw * 1e6).tolist()]
    dev = torch.device("cuda:0")
    params = [{"param": torch.randn(n, device=dev), "grad": torch.randn(n, device=dev).to(torch.bfloat16),
               "exp_avg": torch.zeros(n, device=dev), "exp_avg_sq": torch.zeros(n, device=dev)} for n in sizes]
    hp = dict(lr=3e-4, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1)
    for s in range(args.warmup):
        nsm.adamw_step(params, step=s, **hp)
    torch.cuda.synchronize()
    cap = 8
    ev = HipEvents(2 * cap)
    stages = (ctypes.c_int32 * cap)()
    work = (ctypes.c_double * cap)()
    nl = (ctypes.c_int32 * cap)()
    tr = _lib.MuonTrace(events=ctypes.cast(ev.arr, ctypes.POINTER(ctypes.c_void_p)),
                        stages=ctypes.cast(stages, ctypes.POINTER(ctypes.c_int32)),
                        work=ctypes.cast(work, ctypes.POINTER(ctypes.c_double)), capacity=cap, count=0,
                        group=1, launches=ctypes.cast(nl, ctypes.POINTER(ctypes.c_int32)))
    ms = bytes_ = 0.0
    launches = 0
    for s in range(args.steps):
        nsm.adamw_step(params, step=args.warmup + s, trace=tr, **hp)
        torch.cuda.synchronize()
        for i in range(min(tr.count, cap)):
            ms += ev.elapsed_ms(2 * i, 2 * i + 1)
            bytes_ += work[i]
            launches += nl[i]
    ev.close()
    gbps = bytes_ / (ms * 1e-3) / 1e9
    print(json.dumps({"metric": "AdamW GB/s (vector parameters)", "value": gbps, "unit": "GB/s",
                      "higher_is_better": True, "tensors": len(sizes), "elements": sum(sizes),
                      "ms_per_step": ms / args.steps, "launches_per_step": launches / args.steps,
                      "bytes_per_step": bytes_ / args.steps, "frac_of_hbm": gbps / PEAK_HBM_GBPS,
                      "grad_dtype": "bf16", "data": "synthetic"}), flush=True)


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch loaded (same SONAME)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(h), 0)
            if rc != 0:
                raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)
            self.arr[i] = h
        self.n = n

    def elapsed_ms(self, i, j):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[i], self.arr[j])
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.arr[i])


def setup(w, variant, device, mona_lite=False):
    import torch
    from workloads import make_grads, make_state
    gen_dev = device if w.name.startswith("gram_tall") else "cpu"
    state = make_state(w, device=gen_dev, mona="lite" if (mona_lite and w.mona) else None)
    grads = make_grads(w, step=1, device=gen_dev)
    params = []
    for st, g in zip(state, grads):
        p = {k: v.to(device) for k, v in st.items()}
        p["grad"] = g.to(device)
        params.append(p)
    torch.cuda.synchronize()
    return params


def step_kwargs(w, variant, device="cpu"):
    divisor, restart = w.settings_for(variant)
    kw = dict(lr=w.lr, mu=w.mu, beta_a=w.beta_a, alpha=w.alpha, weight_decay=w.weight_decay,
              ns_steps=w.ns_steps, variant=variant, ns_dtype=w.ns_dtype_for(variant), divisor=divisor,
              restart_every=restart)
    if variant == "limuon":
        from workloads import workload_sketch
        kw.update(w.limuon_settings())
        kw["sketch"] = workload_sketch(w, 1, device=device)
    return kw


def coeff_table(w):
    base = {"cubic": (1.5, -0.5, 0.0), "quintic": (15.0 / 8.0, -5.0 / 4.0, 3.0 / 8.0)}[w.coeffs]
    return [list(base)] * w.ns_steps


def _sysfs_device_dir(dev_index=0):
    """The sysfs directory of the PCI device behind torch's device
    ``dev_index`` (matched by PCI domain/bus/device), or None."""
    import torch
    props = torch.cuda.get_device_properties(dev_index)
    bus = getattr(props, "pci_bus_id", None)
    if bus is None:
        return None
    dom = getattr(props, "pci_domain_id", 0) or 0
    devn = getattr(props, "pci_device_id", 0) or 0
    path = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (dom, bus, devn)
    return path if os.path.isdir(path) else None


def _read_sclk_mhz(path):
    """Current shader clock from the kernel driver's pp_dpm_sclk table (the
    level marked with '*'), read in this process (no child program)."""
    with open(path) as f:
        for line in f:
            if "*" in line:
                digits = "".join(ch for ch in line.split(":", 1)[-1] if ch.isdigit() or ch == ".")
                return float(digits) if digits else None
    return None


def sample_sclk(run, step_ms, seconds=1.0):
    """Shader clock (MHz) while `run` (one step of about `step_ms`) is
    replayed back to back for about `seconds` (about 50 ms of steps queued
    between synchronisations, so the device never idles): the median of the
    driver's current-level readings from sysfs (pp_dpm_sclk), polled by a
    thread of this process.  Returns (MHz or None, reason when None)."""
    import statistics
    import threading
    import torch
    try:
        d = _sysfs_device_dir(torch.cuda.current_device())
    except Exception as e:  # pragma: no cover - depends on the box
        return None, "no PCI address for the device (%s)" % e
    path = os.path.join(d, "pp_dpm_sclk") if d else None
    if path is None or not os.path.exists(path):
        return None, "pp_dpm_sclk not found in sysfs for this device"
    try:
        _read_sclk_mhz(path)
    except OSError as e:
        return None, "pp_dpm_sclk not readable (%s)" % e
    samples = []
    stop = threading.Event()

    def poll():
        while not stop.is_set():
            try:
                v = _read_sclk_mhz(path)
                if v:
                    samples.append(v)
            except OSError:
                return
            time.sleep(0.01)

    batch = max(1, min(1024, int(50.0 / max(step_ms, 1e-3))))
    for _ in range(batch):   # the queue is busy before the first sample
        run()
    th = threading.Thread(target=poll, daemon=True)
    t_end = time.perf_counter() + seconds
    th.start()
    while time.perf_counter() < t_end:
        for _ in range(batch):
            run()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    if not samples:
        return None, "pp_dpm_sclk marked no current level"
    return statistics.median(samples), None


def gpu_timing(args, w, variant):
    import torch
    import newton_schulz_matrix_momentum_amd as nsm
    from newton_schulz_matrix_momentum_amd import _lib

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    params = setup(w, variant, dev, args.mona_lite)
    kw = step_kwargs(w, variant)
    if "sketch" in kw:
        kw["sketch"] = kw["sketch"].to(dev)
    coeffs = coeff_table(w)
    # MONA workloads time steps after the first (D = G - G_prev is live)
    step_idx = 1 if w.mona else 0

    def one_step():
        nsm.muon_step(params, coeffs=coeffs, step=step_idx, **kw)

    for _ in range(max(args.warmup, 1)):
        one_step()
    torch.cuda.synchronize()

    graph = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            one_step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()

    run = graph.replay if graph is not None else one_step
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        run()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / args.steps

    # spread over single steps (outside the timed region): p10 / p50 / p90
    n_dist = min(args.steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_dist)]
    for a, b in evs:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    dist = sorted(a.elapsed_time(b) for a, b in evs)
    spread = [dist[int(q * (n_dist - 1) + 0.5)] for q in (0.1, 0.5, 0.9)]
    # shader clock under the same load (outside the timed region)
    sclk = sample_sclk(run, ms_per_step)

    # MONA workloads: the first step (D = 0: no previous gradient is read)
    # timed on its own graph
    first_ms = None
    if w.mona and graph is not None:
        def step0():
            nsm.muon_step(params, coeffs=coeffs, step=0, **kw)
        s0 = torch.cuda.Stream()
        s0.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s0):
            step0()
        torch.cuda.current_stream().wait_stream(s0)
        torch.cuda.synchronize()
        g0 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g0):
            step0()
        g0.replay()
        torch.cuda.synchronize()
        n0 = max(1, min(args.steps, 20))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n0):
            g0.replay()
        b.record()
        torch.cuda.synchronize()
        first_ms = a.elapsed_time(b) / n0

    # kernel durations: HIP events recorded by libmuon on the launch stream
    # around every run of consecutive launches of one stage (no event between
    # the launches of a run, so the events do not separate the kernels)
    tsteps = args.trace_steps or args.steps
    cap = 512
    ev = HipEvents(2 * cap)
    stages = (ctypes.c_int32 * cap)()
    work = (ctypes.c_double * cap)()
    nl = (ctypes.c_int32 * cap)()
    trace = _lib.MuonTrace(events=ctypes.cast(ev.arr, ctypes.POINTER(ctypes.c_void_p)),
                           stages=ctypes.cast(stages, ctypes.POINTER(ctypes.c_int32)),
                           work=ctypes.cast(work, ctypes.POINTER(ctypes.c_double)), capacity=cap, count=0,
                           group=1, launches=ctypes.cast(nl, ctypes.POINTER(ctypes.c_int32)))
    per_stage = {}
    launches_per_step = 0
    for _ in range(tsteps):
        nsm.muon_step(params, coeffs=coeffs, step=step_idx, trace=trace, **kw)
        torch.cuda.synchronize()
        n = min(trace.count, cap)
        launches_per_step = sum(nl[i] for i in range(n))
        for i in range(n):
            name = _lib.STAGE_NAMES[stages[i]]
            d = per_stage.setdefault(name, {"ms": 0.0, "work": 0.0, "launches": 0})
            d["ms"] += ev.elapsed_ms(2 * i, 2 * i + 1)
            d["work"] += work[i]
            d["launches"] += nl[i]
    ev.close()
    for d in per_stage.values():
        d["ms"] /= tsteps
        d["work"] /= tsteps
        d["launches"] /= tsteps
    return params, ms_per_step, wall, per_stage, launches_per_step, graph is not None, spread, first_ms, sclk


def cpu_baseline(args, w, variant, params, single_thread=False, seconds=None):
    """The oracle as it stands, on this host's cores (or one BLAS thread), on
    a bounded sample: one matrix of each shape class (for the tall-matrix
    Gram set: one per orientation), each repeated until its share of the time
    budget is spent; the per-step time is extrapolated by matrix counts.
    The host BLAS runs one thread per core of this process's affinity mask
    (``cores``)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    import oracle
    affinity = len(os.sched_getaffinity(0))
    threads = 1 if single_thread else affinity
    with threadpool_limits(limits=threads, user_api="blas"):
        blas = max([t.get("num_threads", 1) for t in threadpool_info() if t.get("user_api") == "blas"] or [1])
        divisor, restart = w.settings_for(variant)
        coeffs = oracle.coefficient_table(w.coeffs, w.ns_steps)
        lm = {}
        if variant == "limuon":
            kw = step_kwargs(w, variant)
            lm = dict(rank=kw["rank"], power_iters=kw["power_iters"])
            sketch = kw["sketch"].double().numpy()
        classes = {}
        for i, (r, c) in enumerate(w.shapes):
            classes.setdefault((r, c), []).append(i)
        budget = (args.cpu_seconds if seconds is None else seconds) / max(len(classes), 1)
        total_ms = 0.0
        sample = []
        extrapolated = False
        for (r, c), idx in classes.items():
            p = params[idx[0]]
            snap = {k: v.detach().cpu().double().numpy() for k, v in p.items() if hasattr(v, "detach")}
            if lm:
                lm["omega"] = sketch[:, :max(r, c)].T
            reps, spent = 0, 0.0
            while spent < budget or reps == 0:
                t0 = time.perf_counter()
                oracle.muon_step_matrix(snap["weight"], snap["grad"], snap["momentum"], lr=w.lr, mu=w.mu,
                                        weight_decay=w.weight_decay, coeffs=coeffs, variant=variant,
                                        divisor=divisor, restart_every=restart, accel=snap.get("accel"),
                                        prev_grad=snap.get("prev_grad"), lite_state=snap.get("mona_lite"),
                                        beta_a=w.beta_a, alpha=w.alpha, step=1 if w.mona else 0, **lm)
                spent += time.perf_counter() - t0
                reps += 1
            per = spent / reps
            total_ms += 1e3 * per * len(idx)
            extrapolated = extrapolated or len(idx) > 1
            sample.append("%dx%d: 1 matrix x %d reps, %.2f s each, x%d matrices" % (r, c, reps, per, len(idx)))
            del snap
    return {"value": total_ms, "unit": "ms", "cores": int(threads), "kind": "oracle",
            "affinity_cores": affinity, "blas_threads": int(blas), "extrapolated": extrapolated,
            "sample": "fp64 numpy oracle (full products, no symmetric halving) on one matrix per shape class: " +
                      "; ".join(sample) + ("; per-step time extrapolated by matrix count" if extrapolated else "")}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: libmuon has no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    from workloads import WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(args)
        return
    if args.adamw:
        adamw_probe(args)
        return
    w = WORKLOADS[args.workload]
    if args.grad_kind and args.grad_kind != w.grad_kind:
        import dataclasses
        w = dataclasses.replace(w, grad_kind=args.grad_kind)
    variant = args.variant or w.variants[0]
    print("bench: workload %s variant %s, %d matrices, %s gradients, %d warmup + %d timed steps" %
          (w.name, variant, len(w.shapes), w.grad_kind, args.warmup, args.steps), file=sys.stderr, flush=True)
    params, ms, wall, per_stage, launches, graphed, spread, first_ms, sclk = gpu_timing(args, w, variant)
    print("bench: gpu timing done (%.4f ms/step)" % ms, file=sys.stderr, flush=True)

    gemm = per_stage.get("gemm", {"ms": 0.0, "work": 0.0, "launches": 0})
    ew = [per_stage[k] for k in ("e1", "e2", "e3") if k in per_stage]
    ew_ms = sum(d["ms"] for d in ew)
    ew_bytes = sum(d["work"] for d in ew)
    ns_tflops = gemm["work"] / (gemm["ms"] * 1e-3) / 1e12 if gemm["ms"] > 0 else 0.0
    ew_gbps = ew_bytes / (ew_ms * 1e-3) / 1e9 if ew_ms > 0 else 0.0
    ns_dtype = w.ns_dtype_for(variant)
    peak = PEAK_TFLOPS[ns_dtype]
    # dominant kernel by time per step
    dom = max(per_stage.items(), key=lambda kv: kv[1]["ms"])[0]
    if dom == "gemm" and variant == "limuon":
        # LiMuon's product launches (fp32, against k + p-wide panels) are
        # bound by reading X and updating W, not by MFMA: algorithmic bytes
        # are X read by the 2 + 2q products against it and W read + written
        q = w.limuon_settings()["power_iters"]
        step_bytes = w.numel * (4.0 * (2 + 2 * q) + 8.0)
        per_launch_ms = gemm["ms"] / gemm["launches"]
        per_launch_work = step_bytes / gemm["launches"]
        roof = {"kernel": "LiMuon product launches (fp32 thin products against X, panel updates, weight "
                          "update; all %g launches of a step, averaged)" % gemm["launches"], "bound": "hbm",
                "achieved": per_launch_work / (per_launch_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "avg_launch_us": per_launch_ms * 1e3, "work_per_launch": per_launch_work, "traffic": None}
    elif dom == "gemm":
        per_launch_work = gemm["work"] / gemm["launches"]
        per_launch_ms = gemm["ms"] / gemm["launches"]
        roof = {"kernel": "Newton-Schulz products (%s; all %g product launches of a step, averaged)"
                          % (ns_dtype, gemm["launches"]), "bound": "mfma",
                "achieved": per_launch_work / (per_launch_ms * 1e-3) / 1e12, "peak": peak, "unit": "TFLOP/s",
                "avg_launch_us": per_launch_ms * 1e3, "work_per_launch": per_launch_work,
                "traffic": recorded_traffic(w.name if variant == w.variants[0] else "%s_%s" % (w.name, variant))}
    else:
        d = per_stage[dom]
        per_launch_work = d["work"] / d["launches"]
        per_launch_ms = d["ms"] / d["launches"]
        roof = {"kernel": dom, "bound": "hbm", "achieved": per_launch_work / (per_launch_ms * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "avg_launch_us": per_launch_ms * 1e3,
                "work_per_launch": per_launch_work, "traffic": None}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if roof["bound"] == "mfma":
        # the MFMA peak scales with the shader clock: also quote the fraction
        # of the peak at the clock measured under this load (2.4 GHz nominal)
        mhz, why = sclk
        roof["sclk_mhz"] = mhz
        roof["frac_at_sclk"] = roof["frac"] * SCLK_NOMINAL_MHZ / mhz if mhz else None
        if mhz is None:
            roof["sclk_unavailable"] = why

    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, w, variant, params)
        print("bench: cpu baseline done", file=sys.stderr, flush=True)
        if w.numel <= 4 * 2**20:   # the small sets: also one BLAS thread
            cpu1 = cpu_baseline(args, w, variant, params, single_thread=True, seconds=args.cpu_seconds / 2)
            print("bench: single-thread cpu baseline done", file=sys.stderr, flush=True)

    out = {
        "metric": METRIC,
        "value": ms,
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ns_dtype,
        "data": "synthetic",
        "config": {"workload": w.name + ("+mona_lite" if args.mona_lite and w.mona else ""), "matrices": len(w.shapes),
                   "params": w.numel, "variant": variant,
                   "ns_steps": w.ns_steps, "coeffs": w.coeffs, "grad_dtype": w.grad_dtype, "grads": w.grad_kind,
                   "ns_dtype": ns_dtype,
                   "mona": ("lite" if args.mona_lite else True) if w.mona else False, "hip_graph": graphed, "parallelism": "single_gpu"},
        "ns_tflops": ns_tflops,
        "ns_frac_of_peak": ns_tflops / peak,
        "elementwise_gbps": ew_gbps,
        "elementwise_frac_of_hbm": ew_gbps / PEAK_HBM_GBPS,
        "launches_per_step": launches,
        "stages": {k: {"us_per_step": v["ms"] * 1e3, "launches": v["launches"], "work": v["work"]}
                   for k, v in per_stage.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
        "wall_s_timed": wall,
        "step_ms_p10_p50_p90": spread,
    }
    if first_ms is not None:
        out["first_step_ms"] = first_ms   # MONA: step 0 (no previous gradient read)
    if cpu1 is not None:
        out["cpu_baseline_single_thread"] = cpu1
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
