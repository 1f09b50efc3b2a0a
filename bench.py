"""Benchmark of the chunkwise gated delta rule forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS]
                    [--workloads all|headline] [--no-cpu-baseline]
    python bench.py --counters WORKLOAD:OP      (for rocprofv3 --pmc runs)
    python bench.py --collect-counters DIR [--only SPEC ...]
                                                (runs those rocprofv3 passes, then ingests)
    python bench.py --ingest-counters DIR       (CPU only: counter CSVs -> profiles/)

One step = one gdr_chunk_fwd call over the headline workload (Gated
DeltaNet, bf16 q/k/v/o, fp32 gates and state, B=8 H=16 T=4096 d=128, C=64):
every per-chunk operation of the chunk algorithm runs inside that one kernel.
Inputs are generated on the CPU (seeded) and copied to HBM before timing.
Each workload's step first runs back to back for --settle-ms milliseconds
(untimed; from idle the shader clock takes tens of milliseconds of load to
reach its sustained value), then W untimed warm-up steps; then K steps are
timed between torch.cuda.synchronize() calls, and a pair of HIP events on
the launch stream around them gives the kernel's own average duration, from
which the roofline fraction is computed against the algorithmic bytes
(every input read once, every output written once).

The other workloads are timed the same way and reported under "workloads":
the other four of the pages' configurations (KDA, Q-Delta, Gated DeltaNet-2
and its decode step, the small fp32 case), and the paths beyond them: fp32
I/O at d = 128, the multi-token recurrent form beside the chunk form at T =
16 and 64, the RMSNorm + SiLU output epilogue, and the backward.  A 2 GiB
device copy gives the measured HBM ceiling.  The float64 oracle runs on every
host core (heads split over processes) on a bounded prefix of each workload,
under "cpu_baseline".  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import sys
import time
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunked gated-delta fwd tokens/s and % bf16 MFMA peak, d=128, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2516.6  # 256 CU x 4096 flop/clk x 2.4 GHz, dense
FP32_PEAK_TFLOPS = 157.3        # fp32 on the matrix cores (and the vector ALUs), dense: 256 CU x 256 flop/clk x 2.4 GHz
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "gated_delta_rule_17_amd", "csrc")
CALIB_BYTES = 2 << 30           # device copy that calibrates the HBM counters


def kernel_source_hash() -> str:
    """Hash of every kernel and host source of the library: counter data is
    used only while the sources it was taken with are unchanged."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*.h*")) + glob.glob(os.path.join(CSRC, "*.inc")) +
                       glob.glob(os.path.join(CSRC, "*.cpp"))):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode())
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


def bwd_flops_per_token_head(dk, dv, C=64):
    """Algorithmic flops of the chunk backward per token and head, as the
    passes compute it: the record pass's forward (T, A_qk, the inverse,
    E_bar S, A R, K_tail^T W), then dW = A_qk^T dO + K_tail dS, dR = A^T dW,
    the state gradient's Q_gamma^T dO and E_bar^T dR, the products over the
    value channels (dT, dA_qk, dE_bar, dQ_gamma, dK_tail) and the four
    decay-weighted sums back to the rows (D1 K, D2 K, D1^T E, D2^T Q);
    triangular products count only their non-zero half."""
    full = 2 * C * dk * dv             # a C x dk by dk x dv product (or any of its transposes)
    low_v, low_k = C * (C + 1) * dv, C * (C + 1) * dk   # triangular (diagonal kept) C x C times C x n
    slow_v, slow_k = C * (C - 1) * dv, C * (C - 1) * dk  # strictly triangular
    f = (slow_k + low_k + C * (C - 1) * (C - 2) / 3    # T, A_qk, (I + T)^{-1}
         + 8 * full                                     # E_bar S, K_tail^T W, K_tail dS, Q_gamma^T dO,
                                                        # E_bar^T dR, dE_bar, dQ_gamma, dK_tail
         + 4 * low_v + slow_v                           # A R, A_qk^T dO, A^T dW, dA_qk; dT
         + 2 * slow_k + 2 * low_k)                      # D1 K, D1^T E; D2 K, D2^T Q
    return f / C


def recurrent_flops_per_token_head(dk, dv):
    """Token loop: decay, prediction, write and readout, 2 flop each per state entry."""
    return 8 * dk * dv


# ---- workloads ----------------------------------------------------------------

def workload_list(which):
    """(name, op, config) in bench order; the headline first."""
    from synth import CONFIGS, DECODE, HEADLINE, config
    out = [(HEADLINE, "chunk", config(HEADLINE))]
    if which == "headline":
        return out
    for name in CONFIGS:
        if name != HEADLINE:
            out.append((name, "step" if name == DECODE else "chunk", config(name)))
    out += [
        # fp32 I/O at d = 128 (the plain fp32 kernel's two-pass form: per-chunk prep, then
        # the recurrence on the matrix cores)
        ("gdn_f32_b8h16t4096d128", "chunk", config(HEADLINE, io="f32")),
        # short sequences: the recurrent form beside the chunk form
        ("gdn_bf16_b64h32t4d128", "recurrent", config(HEADLINE, B=64, H=32, T=4)),
        ("gdn_bf16_b64h32t4d128", "chunk", config(HEADLINE, B=64, H=32, T=4)),
        ("gdn_bf16_b64h32t16d128", "recurrent", config(HEADLINE, B=64, H=32, T=16)),
        ("gdn_bf16_b64h32t16d128", "chunk", config(HEADLINE, B=64, H=32, T=16)),
        ("gdn_bf16_b64h32t64d128", "recurrent", config(HEADLINE, B=64, H=32, T=64)),
        ("gdn_bf16_b64h32t64d128", "chunk", config(HEADLINE, B=64, H=32, T=64)),
        # the output epilogue alone over the headline's readout
        ("gdn_bf16_b8h16t4096d128", "epilogue", config(HEADLINE, epilogue=True)),
        # the backward of the headline workload
        ("gdn_bf16_b8h16t4096d128", "bwd", config(HEADLINE)),
    ]
    return out


def algorithmic_bytes(inp, op):
    """Bytes of one call: every input read once, every output written once."""
    q, v = inp["q"], inp["v"]
    B, T, H, dk = q.shape
    dv = v.shape[3]
    io = q.element_size()
    n = B * T * H
    st = B * H * dk * dv * 4
    if op == "epilogue":
        return 3 * n * dv * io + dv * 4          # o, gate in; y out; weight
    gates = sum(inp[key].numel() * 4 for key in ("g", "beta", "b", "w", "lam") if inp[key] is not None)
    fwd_in = n * (2 * dk + dv) * io + gates + (st if inp["state"] is not None else 0)
    if op == "bwd":
        # inputs and the two cotangents in; fp32 gradients of every input out
        grads = n * (2 * dk + dv) * 4 + gates + st
        return fwd_in + n * dv * io + st + grads
    return fwd_in + n * dv * io + st              # + o and the final state out


def bench_workload(name, op, cfg, steps, warmup, settle_ms=0.0):
    import ctypes

    import torch

    import gated_delta_rule_17_amd as gdr
    from gated_delta_rule_17_amd import _lib
    from synth import make_inputs

    inp = make_inputs(cfg)
    dev = torch.device("cuda:0")
    B, T, H = cfg["B"], cfg["T"], cfg["H"]
    # Two copies of every buffer, used alternately, so that a launch finds
    # none of its inputs in the 256 MB last-level cache from the launch before.
    copies = []
    plan = {}
    for _ in range(2):
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        dk, dv = d["k"].shape[3], d["v"].shape[3]
        kinds = dict(decay=d["decay"], erase=d["erase"], write=d["write"], qmix=d["qmix"])
        gates = dict(g=d["g"], beta=d["beta"], b=d["b"], w=d["w"], lam=d["lam"], state=d["state"])
        keep = [d]
        if op == "epilogue":
            o = (torch.randn(B, T, H, dv, device=dev) * 0.05).to(d["q"].dtype)
            a = gdr.GdrNormArgs()
            a.struct_size = ctypes.sizeof(gdr.GdrNormArgs)
            a.dv, a.io, a.eps, a.rows = dv, gdr.DTYPES[o.dtype], 0.0, B * T * H
            y = torch.empty_like(o)
            a.o, a.gate, a.y = o.data_ptr(), d["gate"].data_ptr(), y.data_ptr()
            a.weight = ctypes.cast(ctypes.c_void_p(d["norm_weight"].data_ptr()), ctypes.POINTER(ctypes.c_float))
            keep += [o, y]
            entry, args = "gdr_output_norm_gate", a
        elif op == "bwd":
            do = torch.randn(B, T, H, dv, device=dev).to(d["q"].dtype)
            dS = torch.randn(B, H, dk, dv, device=dev) * 0.1
            fa = gdr.build_args(d["q"], d["k"], d["v"], o=do, **gates, **kinds)
            f32 = dict(dtype=torch.float32, device=dev)
            grads = {"dq": torch.empty(B, T, H, dk, **f32), "dk": torch.empty(B, T, H, dk, **f32),
                     "dv": torch.empty(B, T, H, dv, **f32), "dstate": torch.empty(B, H, dk, dv, **f32)}
            for key, src in (("dg", d["g"]), ("db", d["b"]), ("dw", d["w"]), ("dlam", d["lam"])):
                if src is not None:
                    grads[key] = torch.empty(src.shape, **f32)
            if d["beta"] is not None:
                grads["dbeta"] = torch.empty(B, T, H, **f32)
            need = gdr.bwd_workspace_size(d["q"], d["k"], d["v"], do, **gates, **kinds)
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            args = gdr.build_bwd_args(fa, do, dstate=dS, grads=grads, workspace=ws)
            keep += [do, dS, fa, grads, ws]
            entry = "gdr_chunk_bwd"
            # record pass (prep, recurrence), state, product, key (+ a per-head lambda's reduction)
            plan = dict(workspace_bytes=need, passes=5 + (d["qmix"] == 1))
        else:
            o = torch.empty((B, T, H, dv), dtype=d["q"].dtype, device=dev)
            so = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
            ws = gdr.new_workspace(d["q"], d["k"], d["v"], **gates, **kinds) if op == "chunk" else None
            args = gdr.build_args(d["q"], d["k"], d["v"], o=o, state_out=so, workspace=ws, **gates, **kinds)
            keep += [o, so, ws]
            entry = {"chunk": "gdr_chunk_fwd", "step": "gdr_recurrent_step", "recurrent": "gdr_recurrent_fwd"}[op]
            plan = gdr.plan(d["q"], d["k"], d["v"], op=op, workspace=ws, **gates, **kinds)
            plan["workspace_bytes"] = ws.numel() if ws is not None else 0
        copies.append((keep, args))
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    turn = [0]

    def fn():
        _lib.call(entry, copies[turn[0] & 1][1], sp)
        turn[0] += 1

    ms_step, ms_kern = time_launches(fn, stream, steps, warmup, settle_ms)
    dk, dv = inp["k"].shape[3], inp["v"].shape[3]
    byts = algorithmic_bytes(inp, op)
    res = dict(workload=name, op=op, variant=cfg["variant"], B=B, T=T, H=H, dk=dk, dv=dv, io=cfg["io"],
               ms_per_step=ms_step, kernel_ms_avg=ms_kern, tokens_per_s=B * T / (ms_step * 1e-3),
               algorithmic_bytes=byts, hbm_gbs=byts / (ms_kern * 1e-3) / 1e9, plan=plan)
    res["hbm_frac"] = res["hbm_gbs"] / HBM_PEAK_GBS
    if op == "chunk":
        fl = flops_per_token_head(dk, dv) * B * T * H
    elif op in ("recurrent", "step"):
        fl = recurrent_flops_per_token_head(dk, dv) * B * T * H
    elif op == "bwd":
        fl = bwd_flops_per_token_head(dk, dv) * B * T * H
    else:
        fl = None
    if fl is not None:
        # the peak of the arithmetic the kernels run: the backward and the
        # fp32-I/O chunk form multiply on fp32 operands, the bf16 chunk forms on bf16
        fp32 = op == "bwd" or (op == "chunk" and cfg["io"] == "f32")
        peak = FP32_PEAK_TFLOPS if fp32 else MFMA_BF16_PEAK_TFLOPS
        res["algorithmic_flops"] = fl
        res["tflops"] = fl / (ms_kern * 1e-3) / 1e12
        res["peak_tflops"] = peak
        res["mfma_frac"] = res["tflops"] / peak
    if op == "chunk" and T >= 64:
        res["us_per_chunk_step"] = ms_kern * 1e3 / ((T + 63) // 64)
    del copies
    torch.cuda.empty_cache()
    return res, inp


def time_launches(fn, stream, steps, warmup, settle_ms=0.0):
    """Wall time per step and the kernel's average duration per launch.

    Untimed first: the step back to back for ``settle_ms`` milliseconds,
    then ``warmup`` steps.  One pair of HIP events on the launch stream
    brackets the whole timed region: the launches queue back to back, so the
    average is the kernels' own duration plus the small gaps between them.
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


def copy_ceiling(settle_ms=100.0):
    """GB/s of a plain 2 GiB device-to-device copy (reads and writes counted)."""
    import torch
    src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    _, ms = time_launches(lambda: dst.copy_(src), stream, 10, 2, settle_ms)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * CALIB_BYTES / (ms * 1e-3) / 1e9


# ---- the oracle on the host ------------------------------------------------------

def _oracle_worker(args):
    import numpy as np  # noqa: F401  (each worker imports with one BLAS thread)
    from oracle import gdr_recurrence
    sub, kw = args
    t0 = time.perf_counter()
    gdr_recurrence(sub["q"], sub["k"], sub["v"], **kw)
    return time.perf_counter() - t0


def _seq_slice(x, bs, hs, Ts):
    """x [B, T, H, ...] -> [len(pairs), Ts, 1, ...] for the given (b, h) pairs."""
    return x[bs, :Ts, hs][:, :, None] if x.ndim == 3 else x[bs, :Ts, hs, :][:, :, None, :]


def cpu_baseline_all(items, budget_s=3.0):
    """The float64 oracle as it stands, on every core of this host: each
    workload's (batch, head) pairs are split over one process per core (one
    BLAS thread each) on a prefix of the tokens sized to about ``budget_s``
    seconds of wall time.  Returns {workload: {...}}."""
    import multiprocessing as mp

    import numpy as np

    cores = len(os.sched_getaffinity(0))
    env = {k: "1" for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    ctx = mp.get_context("spawn")
    out = {}
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    with ctx.Pool(cores) as pool:
        z = np.zeros((1, 1, 1, 4))
        pool.map(_oracle_worker, [({"q": z, "k": z, "v": z}, {"beta": np.ones((1, 1, 1))})] * cores)  # start
        for name, inp in items:
            B, T, H = inp["q"].shape[:3]
            pairs = [(b, h) for b in range(B) for h in range(H)]

            def jobs_for(Ts):
                res = []
                for i in range(min(cores, len(pairs))):
                    part = pairs[i::cores]
                    bs = np.array([p[0] for p in part])
                    hs = np.array([p[1] for p in part])
                    def sl(key):
                        val = inp[key]
                        return None if val is None else _seq_slice(val.float().numpy(), bs, hs, Ts)
                    kw = dict(decay=inp["decay"], g=sl("g"), erase=inp["erase"], write=inp["write"],
                              beta=sl("beta"), b=sl("b"), w=sl("w"), qmix=inp["qmix"], lam=None,
                              state=None if inp["state"] is None else inp["state"].numpy()[bs, hs][:, None])
                    if inp["qmix"]:
                        lam = inp["lam"].float().numpy()
                        kw["lam"] = (np.repeat(lam[hs][:, None], Ts, axis=1)[:, :, None] if lam.ndim == 1
                                     else lam[bs, :Ts, hs][:, :, None])
                    res.append(({"q": sl("q"), "k": sl("k"), "v": sl("v")}, kw))
                return res

            def run(Ts):
                jobs = jobs_for(Ts)
                t0 = time.perf_counter()
                busy = sum(pool.map(_oracle_worker, jobs))
                return time.perf_counter() - t0, busy

            T0 = min(T, 64)
            w0, _ = run(T0)
            Ts = int(min(T, max(T0, budget_s / max(w0, 1e-6) * T0)))
            wall, busy = run(Ts)
            out[name] = dict(value=B * Ts / wall, unit="tokens/s", token_heads_per_s=B * H * Ts / wall,
                             cores=min(cores, len(pairs)), kind="oracle",
                             sample=f"{name}: all {B} batch rows x {H} heads, first {Ts} of {T} tokens, "
                                    f"float64 numpy token loop, (batch, head) pairs split over "
                                    f"{min(cores, len(pairs))} processes, {wall:.2f} s wall, "
                                    f"{busy:.1f} s summed worker time",
                             cpu_model=model)
    for k, v in old.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v
    return out


# ---- counters ----------------------------------------------------------------------

def counters_run(spec):
    """Dispatches for one rocprofv3 --pmc pass: a 2 GiB device copy (the
    calibration: it reads and writes exactly 2 GiB), then three calls of one
    workload's op."""
    import torch
    name, op = spec.split(":")
    src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    for wname, wop, cfg in workload_list("all"):
        if wname == name and wop == op:
            bench_workload(wname, wop, cfg, 3, 0)
            break
    else:
        raise SystemExit(f"unknown workload {spec}")
    torch.cuda.synchronize()
    print(f"counters run done: copy {CALIB_BYTES >> 30} GiB, then 3 calls of {spec}", file=sys.stderr, flush=True)


PMC_PASSES = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "mfma": ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_VALU_MFMA_BUSY_CYCLES",
             "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "GRBM_GUI_ACTIVE"],
}


def collect_counters(outdir, only=None):
    """One rocprofv3 --pmc pass per (workload, op, counter set), each a child
    process `rocprofv3 --pmc ... -- python3 bench.py --counters W:OP` with a
    time limit of its own; this process never touches the GPU.  Then ingest."""
    import subprocess
    outdir = os.path.abspath(outdir)
    os.makedirs(outdir, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    specs = [f"{n}:{o}" for n, o, _ in workload_list("all")]
    if only:
        specs = [s2 for s2 in specs if s2 in only]
    for spec in specs:
        for pas, cnts in PMC_PASSES.items():
            cmd = ["rocprofv3", "--pmc", *cnts, "-f", "csv", "-d", os.path.join(outdir, f"{spec}.{pas}"), "-o", "c",
                   "--", sys.executable, os.path.join(ROOT, "bench.py"), "--counters", spec]
            t0 = time.time()
            r = subprocess.run(["timeout", "-s", "KILL", "240", *cmd], cwd="/tmp", env=env,
                               capture_output=True, text=True)
            ok = "counters run done" in r.stderr
            print(f"# pmc {spec} {pas}: rc {r.returncode} in {time.time() - t0:.0f} s{'' if ok else ' (FAILED)'}",
                  flush=True)
            if not ok:
                print(r.stdout[-2000:], r.stderr[-3000:], file=sys.stderr)
                raise SystemExit(1)
    ingest_counters(outdir)


def _demangle(kname):
    if not kname.startswith("_Z"):
        return kname
    import subprocess
    try:
        # this c++filt does not know the bf16 code DF16b: spell it as a vendor type
        name = kname.replace("DF16b", "u6__bf16")
        return subprocess.run(["c++filt", name], capture_output=True, text=True).stdout.strip() or kname
    except OSError:
        return kname


def _short(kname):
    """Kernel name without namespace and parameter list."""
    k = _demangle(kname).split("(")[0].replace("gdr::", "").replace("void ", "")
    return k.strip()


def ingest_counters(root):
    """CPU only: read the counter CSVs of `root/<workload>.<op>.<pass>/c_counter_collection.csv`
    (pass = fetch, write or mfma), scale the HBM counters by what they read
    for the 2 GiB calibration copy, and write profiles/traffic.json and
    profiles/counters.md."""
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(dict)))  # spec -> kernel -> counter -> [vals]
    calib = {}
    for path in sorted(glob.glob(os.path.join(root, "*", "*counter_collection.csv"))):
        spec_pass = os.path.basename(os.path.dirname(path))
        spec, pas = spec_pass.rsplit(".", 1)
        vals = defaultdict(lambda: defaultdict(float))
        names = {}
        for r in csv.DictReader(open(path)):
            dsp = int(r["Dispatch_Id"])
            # summed over the counter's instances (shader engines, XCDs), and the
            # largest instance (what a cycle count such as GRBM_GUI_ACTIVE needs)
            vals[dsp][r["Counter_Name"]] += float(r["Counter_Value"])
            mk = r["Counter_Name"] + "_max"
            vals[dsp][mk] = max(vals[dsp].get(mk, 0.0), float(r["Counter_Value"]))
            names[dsp] = r["Kernel_Name"]
        copies = [d for d in vals if "copy" in names[d].lower()]
        if pas in ("fetch", "write") and copies:
            cnt = "FETCH_SIZE" if pas == "fetch" else "WRITE_SIZE"
            big = max(copies, key=lambda d: vals[d].get(cnt, 0.0))
            calib[(spec, pas)] = vals[big].get(cnt, 0.0)
        for dsp in sorted(vals):
            if "gdr::" not in names[dsp] and not names[dsp].startswith("_ZN3gdr"):
                continue
            k = _short(names[dsp])
            for cname, v in vals[dsp].items():
                per[spec][k].setdefault(cname, []).append(v)
    data = {"kernel_src_sha": kernel_source_hash(), "calibration_bytes": CALIB_BYTES, "workloads": {}}
    for spec, kernels in per.items():
        ent = {}
        for k, cnts in kernels.items():
            e = {}
            for cname, vs in cnts.items():
                e[cname] = sum(vs) / len(vs)
            e["calls"] = max(len(vs) for vs in cnts.values())
            if "FETCH_SIZE" in e and (spec, "fetch") in calib:
                f = (CALIB_BYTES / 1024) / calib[(spec, "fetch")]
                e["fetch_bytes"] = e["FETCH_SIZE"] * f * 1024
                e["fetch_factor"] = f
            if "WRITE_SIZE" in e and (spec, "write") in calib:
                f = (CALIB_BYTES / 1024) / calib[(spec, "write")]
                e["write_bytes"] = e["WRITE_SIZE"] * f * 1024
                e["write_factor"] = f
            ent[k] = e
        data["workloads"][spec] = ent
    with open(os.path.join(PROFILES, "traffic.json"), "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(f"wrote {os.path.join(PROFILES, 'traffic.json')} ({len(data['workloads'])} workloads)")


def traffic_of(name, op):
    """Measured HBM bytes per call of a workload (summed over its kernels) and
    the per-kernel counter entries, if taken with the current sources."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None, None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None, None
    if data.get("kernel_src_sha") != kernel_source_hash():
        return None, None
    ent = data.get("workloads", {}).get(f"{name}:{op}")
    if not ent:
        return None, None
    tot = 0.0
    for e in ent.values():
        if "fetch_bytes" not in e or "write_bytes" not in e:
            return None, ent
        tot += e["fetch_bytes"] + e["write_bytes"]
    return tot, ent


# ---- main ----------------------------------------------------------------------------

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
    ap.add_argument("--counters", metavar="WORKLOAD:OP",
                    help="for rocprofv3 --pmc runs: one 2 GiB device copy (calibration) and three calls of "
                         "one workload's op, no timing output")
    ap.add_argument("--ingest-counters", metavar="DIR",
                    help="CPU only: turn the counter CSVs under DIR into profiles/traffic.json")
    ap.add_argument("--collect-counters", metavar="DIR",
                    help="run the rocprofv3 --pmc passes of every workload (child processes), then ingest")
    ap.add_argument("--only", nargs="*", help="with --collect-counters: these WORKLOAD:OP specs only")
    ap.add_argument("--list-workloads", action="store_true")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(args.ingest_counters)
        return
    if args.collect_counters:
        collect_counters(args.collect_counters, args.only)
        return
    if args.list_workloads:
        for name, op, _ in workload_list("all"):
            print(f"{name}:{op}")
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the chunked forward shards over (batch, head) with no "
              "exchange, so a multi-GPU figure is not produced here; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    torch.cuda.init()
    if args.counters:
        counters_run(args.counters)
        return
    items = workload_list(args.workloads)
    head_name, _, head_cfg = items[0]
    head, head_inp = bench_workload(head_name, "chunk", head_cfg, args.steps, args.warmup, settle_ms=args.settle_ms)
    print(f"# headline {head_name}: {head['kernel_ms_avg'] * 1e3:.1f} us/launch, "
          f"{head['hbm_gbs']:.0f} GB/s ({head['hbm_frac'] * 100:.1f}% HBM), "
          f"{head['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)

    workloads = {}
    oracle_items = [(f"{head_name}:chunk", head_inp)]
    for name, op, cfg in items[1:]:
        steps = max(5, args.steps // 2) if op != "bwd" else 5
        r, inp = bench_workload(name, op, cfg, steps, args.warmup, settle_ms=args.settle_ms)
        keep = ("op", "tokens_per_s", "kernel_ms_avg", "hbm_gbs", "hbm_frac", "tflops", "peak_tflops", "mfma_frac", "plan",
                "algorithmic_bytes", "us_per_chunk_step")
        ent = {k: r[k] for k in keep if k in r}
        tr, _ = traffic_of(name, op)
        if tr is not None:
            ent["traffic_bytes"] = tr
            ent["traffic_ratio"] = tr / r["algorithmic_bytes"]
        workloads[f"{name}:{op}"] = ent
        if op in ("chunk", "step") and name in ("kda_bf16_b4h32t8192d128", "qdelta_bf16_b8h8t4096d128",
                                                "gdn2_bf16_b1h32t65536d128", "gdn2_decode_b256h32d128",
                                                "gdn_f32_b1h2t256d64"):
            oracle_items.append((f"{name}:{op}", inp))
        print(f"# {name}:{op}: {r['kernel_ms_avg'] * 1e3:.1f} us/call, {r['hbm_gbs']:.0f} GB/s "
              f"({r['hbm_frac'] * 100:.1f}% HBM)", file=sys.stderr, flush=True)

    ceiling = copy_ceiling()
    print(f"# copy ceiling: {ceiling:.0f} GB/s", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        allcpu = cpu_baseline_all(oracle_items)
        cpu = dict(allcpu[f"{head_name}:chunk"])
        cpu["workloads"] = {k: {kk: v[kk] for kk in ("value", "unit", "token_heads_per_s", "cores", "sample")}
                            for k, v in allcpu.items() if k != f"{head_name}:chunk"}
        print(f"# cpu baseline: {cpu['value']:.1f} tokens/s on {cpu['cores']} cores", file=sys.stderr,
              flush=True)

    traffic, kents = traffic_of(head_name, "chunk")
    n_chunks = (head["T"] + 63) // 64
    roof = dict(bound="hbm", achieved=head["hbm_gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                frac=head["hbm_frac"], traffic=traffic,
                traffic_ratio=traffic / head["algorithmic_bytes"] if traffic else None,
                algorithmic_bytes_per_launch=head["algorithmic_bytes"],
                kernel_ms_avg=head["kernel_ms_avg"],
                kernel="pipe_fwd_kernel<128,%d,0,false>" % head["plan"]["dv_slice"],
                copy_ceiling_gbs=ceiling, frac_of_copy_ceiling=head["hbm_gbs"] / ceiling,
                limiter=("latency of the serial chunk steps: each workgroup walks %d dependent chunk steps "
                         "of its (batch, head, value slice); the kernel moves its algorithmic bytes "
                         "(traffic_ratio) at %.0f%% of HBM" % (n_chunks, head["hbm_frac"] * 100)),
                us_per_chunk_step=head["kernel_ms_avg"] * 1e3 / n_chunks)
    if kents:
        for k, e in kents.items():
            if "SQ_VALU_MFMA_BUSY_CYCLES" in e and "GRBM_GUI_ACTIVE" in e:
                # MFMA busy cycles over the 1024 SIMDs' cycles while the kernel
                # ran; rocprofv3 reports GRBM_GUI_ACTIVE summed over the 8 XCDs
                roof["mfma_busy_frac_counter"] = e["SQ_VALU_MFMA_BUSY_CYCLES"] / (e["GRBM_GUI_ACTIVE"] / 8 * 1024)
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
        "config": {"workload": head_name, "variant": "gated_deltanet", "B": head["B"], "T": head["T"],
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
