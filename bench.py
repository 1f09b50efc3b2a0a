"""Benchmark of the chunkwise gated delta rule forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS]
                    [--workloads all|headline] [--no-cpu-baseline]

One step = one gdr_chunk_fwd call over the headline workload (Gated
DeltaNet, bf16 q/k/v/o, fp32 gates and state, B=8 H=16 T=4096 d=128, C=64):
every per-chunk operation of the chunk algorithm runs inside that one kernel.
Inputs are generated on the CPU (seeded) and copied to HBM before timing.
Each workload's step first runs back to back for --settle-ms milliseconds
(untimed; from idle the shader clock takes tens of milliseconds of load to
reach its sustained value), then W untimed warm-up steps; then K steps are
timed between torch.cuda.synchronize() calls, and a pair of HIP events on
the launch stream around them gives the kernel's own average duration, from
which the roofline fraction is computed against the
algorithmic bytes (every input read once, every output written once).

The other workloads (KDA, Q-Delta, Gated DeltaNet-2, and the decode step)
are timed the same way and reported under "workloads"; the float64 oracle
is timed on a bounded sample of the headline workload under "cpu_baseline".
Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import resource
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunked gated-delta fwd tokens/s and % bf16 MFMA peak, d=128, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2516.6  # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["common.hpp", "chunk_kernel.hpp", "pipe_kernel.hpp", "pipe_instances.inc", "pipe_gm0.hip",
                  "step_kernel.hpp", "chunk_instances.inc", "step.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_delta_rule_17_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def flops_per_token_head(dk, dv, C=64):
    """Algorithmic flops of the chunk algorithm per token and head; the
    triangular products count only their non-zero half."""
    f = (C * (C - 1) * dk          # T = tril(E_bar K_bar^T, -1)
         + C * (C + 1) * dk        # A_qk = tril(Q_gamma K_bar^T, 0)
         + C * (C - 1) * (C - 2) / 3  # (I + T)^{-1}
         + C * (C - 1) * dk        # Y = A E_bar
         + C * (C - 1) * dv        # U = A Z
         + 6 * C * dk * dv         # Y S, Q_gamma S, K_tail^T W
         + C * (C + 1) * dv)       # A_qk W
    return f / C


def algorithmic_bytes(cfg, inp, op="chunk"):
    B, T, H = cfg["B"], cfg["T"], cfg["H"]
    dk = inp["k"].shape[3]
    dv = inp["v"].shape[3]
    io = inp["q"].element_size()
    n = B * T * H
    by = n * (2 * dk + 2 * dv) * io   # q, k, v read; o written
    if inp["g"] is not None:
        by += inp["g"].numel() * 4
    for key in ("beta", "b", "w", "lam"):
        if inp[key] is not None:
            by += inp[key].numel() * 4
    st = B * H * dk * dv * 4
    by += st * (2 if inp["state"] is not None else 1)
    return by


def traffic_from_profile(kernel_tag, workload):
    """HBM bytes per launch measured by rocprofv3 counters, if the profile was
    taken with the current kernel sources; else None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = data.get(kernel_tag, {}).get(workload)
    if not ent or ent.get("kernel_src_sha") != kernel_source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


def time_launches(fn, stream, steps, warmup, settle_ms=0.0):
    """Wall time per step and the kernel's average duration per launch.

    Untimed first: the step back to back for ``settle_ms`` milliseconds,
    then ``warmup`` steps.  From idle the GPU raises its shader clock over
    some tens of milliseconds of load, so steps timed right after a few
    warm-up launches measure the ramp rather than the clock that sustained
    load runs at.

    One pair of HIP events on the launch stream brackets the whole timed
    region: the launches queue back to back, so the average is the kernel's
    own duration plus the small gaps between consecutive kernels.  (An event
    pair around every launch would add the event packets' own gaps to each.)
    """
    import torch
    t_end = time.perf_counter() + settle_ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall / steps * 1e3, e0.elapsed_time(e1) / steps


def bench_workload(name, steps, warmup, op="chunk", settle_ms=0.0):
    import ctypes

    import torch

    import gated_delta_rule_17_amd as gdr
    from gated_delta_rule_17_amd import _lib
    from synth import config, make_inputs

    cfg = config(name)
    inp = make_inputs(cfg)
    dev = torch.device("cuda:0")
    B, T, H = cfg["B"], cfg["T"], cfg["H"]
    # Two copies of every buffer, used alternately, so that a launch finds
    # none of its inputs in the 256 MB last-level cache from the launch before.
    copies = []
    for _ in range(2):
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        dk, dv = d["k"].shape[3], d["v"].shape[3]
        o = torch.empty((B, T, H, dv), dtype=d["q"].dtype, device=dev)
        so = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        kinds = dict(decay=d["decay"], erase=d["erase"], write=d["write"], qmix=d["qmix"])
        gates = dict(g=d["g"], beta=d["beta"], b=d["b"], w=d["w"], lam=d["lam"], state=d["state"])
        # the two-pass per-channel form, where the library offers one, with
        # its workspace (one per copy, like every other buffer)
        ws = gdr.new_workspace(d["q"], d["k"], d["v"], **gates, **kinds) if op == "chunk" else None
        args = gdr.build_args(d["q"], d["k"], d["v"], o=o, state_out=so, workspace=ws, **gates, **kinds)
        copies.append((d, o, so, args, ws))
    d = copies[0][0]
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    entry = "gdr_chunk_fwd" if op == "chunk" else "gdr_recurrent_step"
    plan = gdr.plan(d["q"], d["k"], d["v"], op=op, g=d["g"], beta=d["beta"], b=d["b"], w=d["w"],
                    lam=d["lam"], state=d["state"], workspace=copies[0][4], **kinds)
    plan["workspace_bytes"] = copies[0][4].numel() if copies[0][4] is not None else 0
    turn = [0]

    def fn():
        _lib.call(entry, copies[turn[0] & 1][3], sp)
        turn[0] += 1

    ms_step, ms_kern = time_launches(fn, stream, steps, warmup, settle_ms)
    byts = algorithmic_bytes(cfg, inp, op)
    tokens = B * T
    res = dict(workload=name, variant=cfg["variant"], B=B, T=T, H=H, dk=dk, dv=dv, io=cfg["io"],
               ms_per_step=ms_step, kernel_ms_avg=ms_kern,
               tokens_per_s=tokens / (ms_step * 1e-3), algorithmic_bytes=byts,
               hbm_gbs=byts / (ms_kern * 1e-3) / 1e9, plan=plan)
    res["hbm_frac"] = res["hbm_gbs"] / HBM_PEAK_GBS
    if op == "chunk":
        fl = flops_per_token_head(dk, dv) * B * T * H
        res["algorithmic_flops"] = fl
        res["tflops"] = fl / (ms_kern * 1e-3) / 1e12
        res["mfma_frac"] = res["tflops"] / MFMA_BF16_PEAK_TFLOPS
    del d, copies
    torch.cuda.empty_cache()
    return res, inp


def cpu_baseline(name, inp, budget_s=15.0):
    """The float64 oracle as it stands, on a bounded prefix of the workload's
    sequences (all batch rows and heads), scaled to tokens/s."""
    from oracle import gdr_recurrence
    from synth import oracle_kwargs

    def run(Ts):
        sub = {}
        for key, val in inp.items():
            if hasattr(val, "dim") and key not in ("lam", "state"):
                sub[key] = val[:, :Ts]
            else:
                sub[key] = val
        r0 = resource.getrusage(resource.RUSAGE_SELF)
        t0 = time.perf_counter()
        gdr_recurrence(sub["q"], sub["k"], sub["v"], **oracle_kwargs(sub))
        wall = time.perf_counter() - t0
        r1 = resource.getrusage(resource.RUSAGE_SELF)
        cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
        return wall, cpu

    B, T = inp["q"].shape[0], inp["q"].shape[1]
    w64, _ = run(64)
    Ts = int(min(T, max(64, budget_s / max(w64, 1e-6) * 64)))
    wall, cpu = run(Ts)
    cores = max(1, round(cpu / wall))
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return dict(value=B * Ts / wall, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{name}: all {B} batch rows x {inp['q'].shape[2]} heads, first {Ts} of {T} "
                       f"tokens, float64 numpy token loop, {wall:.1f} s wall, {cpu:.1f} s cpu",
                cpu_model=model, host_threads_available=len(os.sched_getaffinity(0)))


def ingest_counters(fetch_csv, write_csv, kernel_tag="pipe_fwd_kernel", workload=None):
    """Write the headline kernel's HBM bytes per launch to profiles/traffic.json
    from the counter CSVs of two `rocprofv3 --pmc` passes over `bench.py
    --counters` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Each counter
    is scaled by what it reads for the 1 GiB device copy that the run makes
    first (the copy reads and writes exactly 1 GiB)."""
    import csv
    from collections import defaultdict

    from synth import HEADLINE

    workload = workload or HEADLINE

    def per_dispatch(path, counter):
        vals, names = defaultdict(float), {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            vals[d] += float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
        copy = [vals[d] for d in sorted(vals) if "copy" in names[d].lower()]
        kern = [vals[d] for d in sorted(vals) if kernel_tag in names[d]]
        if not copy or not kern:
            raise SystemExit(f"{path}: no copy or no {kernel_tag} dispatch with {counter}")
        return copy[0], sum(kern) / len(kern)

    gib_kib = float(1 << 20)
    fcopy, fkern = per_dispatch(fetch_csv, "FETCH_SIZE")
    wcopy, wkern = per_dispatch(write_csv, "WRITE_SIZE")
    ff, wf = gib_kib / fcopy, gib_kib / wcopy
    fetch_b, write_b = fkern * ff * 1024, wkern * wf * 1024
    path = os.path.join(PROFILES, "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data.setdefault(kernel_tag, {})[workload] = {
        "kernel_src_sha": kernel_source_hash(),
        "hbm_bytes_per_launch": fetch_b + write_b,
        "fetch_bytes_per_launch": fetch_b,
        "write_bytes_per_launch": write_b,
        "fetch_kib_raw": fkern,
        "write_kib_raw": wkern,
        "copy_calibration": {"bytes": 1 << 30, "fetch_kib_raw": fcopy, "write_kib_raw": wcopy,
                             "fetch_factor": ff, "write_factor": wf},
    }
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
    print(f"{kernel_tag} {workload}: read {fetch_b / 1e6:.1f} MB, write {write_b / 1e6:.1f} MB per launch "
          f"(factors {ff:.3f}, {wf:.3f}) -> {path}")


def counters_run(name):
    """Dispatches for HBM counter calibration: a plain device-to-device copy of
    exactly 1 GiB (reads 1 GiB, writes 1 GiB), then the headline chunk kernel."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    bench_workload(name, 3, 0)
    torch.cuda.synchronize()
    print(f"counters run done: copy 1 GiB, then 3 launches of {name}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed back-to-back steps before the warm-up steps of each workload, in "
                         "milliseconds, so that the timed steps run at the sustained clock")
    ap.add_argument("--workloads", choices=["all", "headline"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="for rocprofv3 --pmc runs: one 1 GiB device copy (calibration) and three "
                         "launches of the headline chunk kernel, no timing output")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="CPU only: turn the counter CSVs of the FETCH_SIZE and WRITE_SIZE passes over "
                         "--counters into profiles/traffic.json")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the chunked forward shards over (batch, head) with no "
              "exchange, so a multi-GPU figure is not produced here; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from synth import CONFIGS, DECODE, HEADLINE

    torch.cuda.init()
    if args.counters:
        counters_run(HEADLINE)
        return
    head, head_inp = bench_workload(HEADLINE, args.steps, args.warmup, settle_ms=args.settle_ms)
    print(f"# headline {HEADLINE}: {head['kernel_ms_avg'] * 1e3:.1f} us/launch, "
          f"{head['hbm_gbs']:.0f} GB/s ({head['hbm_frac'] * 100:.1f}% HBM), "
          f"{head['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)

    workloads = {}
    if args.workloads == "all":
        for name in CONFIGS:
            if name == HEADLINE:
                continue
            op = "step" if name == DECODE else "chunk"
            r, _ = bench_workload(name, max(5, args.steps // 2), args.warmup, op=op, settle_ms=args.settle_ms)
            keep = ("tokens_per_s", "kernel_ms_avg", "hbm_gbs", "hbm_frac", "tflops", "mfma_frac", "plan",
                    "algorithmic_bytes")
            workloads[name] = {k: r[k] for k in keep if k in r}
            print(f"# {name}: {r['kernel_ms_avg'] * 1e3:.1f} us/launch, {r['hbm_gbs']:.0f} GB/s "
                  f"({r['hbm_frac'] * 100:.1f}% HBM)", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(HEADLINE, head_inp)
        print(f"# cpu baseline: {cpu['value']:.1f} tokens/s on {cpu['cores']} cores", file=sys.stderr,
              flush=True)

    traffic = traffic_from_profile("pipe_fwd_kernel", HEADLINE)
    roof = dict(bound="hbm", achieved=head["hbm_gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                frac=head["hbm_frac"], traffic=traffic,
                algorithmic_bytes_per_launch=head["algorithmic_bytes"],
                kernel_ms_avg=head["kernel_ms_avg"], kernel="pipe_fwd_kernel<128,%d,0,false>" % head["plan"]["dv_slice"])
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "variant": "gated_deltanet", "B": head["B"], "T": head["T"],
                   "H": head["H"], "dk": head["dk"], "dv": head["dv"], "chunk": 64,
                   "io": "bf16 q/k/v/o, fp32 gates and state", "dv_slice": head["plan"]["dv_slice"],
                   "grid": head["plan"]["grid"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "tflops": head["tflops"],
        "mfma_frac": head["mfma_frac"],
        "workloads": workloads,
        "kernel_src_sha": kernel_source_hash(),
        "host": platform.node(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
