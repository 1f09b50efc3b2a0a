"""Helpers shared by the GPU tests (imported only by test modules)."""

import sys

import numpy as np
import torch

import gated_delta_rule_17_amd as gdr
from oracle import gdr_recurrence
from synth import make_inputs, oracle_kwargs, rel_err

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(inp, dev="cuda:0"):
    out = {}
    for key, val in inp.items():
        out[key] = val.to(dev) if isinstance(val, torch.Tensor) else val
    return out


def gpu_kwargs(d):
    return dict(g=d["g"], beta=d["beta"], b=d["b"], w=d["w"], lam=d["lam"], state=d["state"],
                decay=d["decay"], erase=d["erase"], write=d["write"], qmix=d["qmix"])


def run_chunk(inp, dv_split=0, two_pass=None):
    d = to_dev(inp)
    o, S = gdr.chunk_fwd(d["q"], d["k"], d["v"], dv_split=dv_split, two_pass=two_pass, **gpu_kwargs(d))
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy()


def run_oracle(inp, heads=None):
    """Oracle on all heads, or on a list of (b, h) pairs (each a full
    sequence; run as one batch of single-head sequences)."""
    if heads is None:
        return gdr_recurrence(inp["q"], inp["k"], inp["v"], **oracle_kwargs(inp))
    bs = torch.tensor([b for b, _ in heads])
    hs = torch.tensor([h for _, h in heads])
    sub = {}
    for key, val in inp.items():
        if not isinstance(val, torch.Tensor):
            sub[key] = val
        elif key == "lam":
            sub[key] = val[hs] if val.dim() == 1 else val[bs, :, hs][:, :, None]
        elif key == "state":
            sub[key] = val[bs, hs][:, None]
        elif key in ("gate", "norm_weight"):
            continue
        else:
            sub[key] = val[bs, :, hs][:, :, None] if val.dim() == 3 else val[bs, :, hs, :][:, :, None, :]
    kw = oracle_kwargs(sub)
    if sub["qmix"] and inp["lam"].dim() == 1:
        # a per-head lambda: every sampled pair is its own batch row of one head
        kw["lam"] = sub["lam"][:, None].expand(len(heads), sub["q"].shape[1]).unsqueeze(-1).contiguous()
    o, S = gdr_recurrence(sub["q"], sub["k"], sub["v"], **kw)
    return [o[i, :, 0] for i in range(len(heads))], [S[i, 0] for i in range(len(heads))]


def elementwise_rel(x, ref):
    """Diagnostic: max |x - ref| / (|ref| + 1e-6), elementwise."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float((np.abs(x - ref) / (np.abs(ref) + 1e-6)).max())


def assert_parity(name, o, S, o_ref, S_ref, tol):
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    finite = np.isfinite(o).all() and np.isfinite(S).all()
    say(f"    {name}: rel err o {eo:.3e}  S {es:.3e}  (tol {tol:.0e})")
    assert finite, f"{name}: non-finite output"
    assert eo <= tol and es <= tol, f"{name}: o {eo:.3e} S {es:.3e} > {tol:.0e}"
    return eo, es
