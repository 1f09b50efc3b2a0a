"""Seeded synthetic inputs for the gated delta rule workloads.

Shared by the tests, the benchmark and the smoke check.  It holds none of the
method's arithmetic: it draws random tensors and applies the caller-side
input preparation that the pages put outside the operator (L2-normalised q
and k, q optionally scaled by dk^-1/2, sigmoid gates, log-decay
g = -softplus(.) kept in fp32; [GDN2] training strategy and [CH11] §11.3).

Draw order (fixed, one ``torch.Generator`` seeded with the config's seed):
q_raw, k_raw, v, then beta or (b, w), then g, then lambda, then the initial
state.  Each draw is a full-size standard normal (or uniform for lambda) in
fp32; L2 normalisation is over the head dimension in fp32; q, k, v are then
rounded to nearest-even bf16 for bf16 I/O.  The pages measure on trained
models and natural text (FineWeb-Edu, RULER); none of that is available, so
these inputs stand in for trained activations with the pages' shapes.
"""

from __future__ import annotations

import math

import torch

# Workloads.  d = dk = dv.  "decay_shift" c gives g = -softplus(N(0,1) + c).
CONFIGS = {
    # plain Gated DeltaNet at fp32 I/O (the small parity case)
    "gdn_f32_b1h2t256d64": dict(variant="gdn", B=1, H=2, T=256, d=64, io="f32",
                                q_scale=True, decay_shift=2.0, state_std=0.0, seed=0),
    # Gated DeltaNet, bf16 q/k/v/o, fp32 gates and state (the headline workload)
    "gdn_bf16_b8h16t4096d128": dict(variant="gdn", B=8, H=16, T=4096, d=128, io="bf16",
                                    q_scale=True, decay_shift=2.0, state_std=0.01, seed=1),
    # KDA: per-key-channel decay
    "kda_bf16_b4h32t8192d128": dict(variant="kda", B=4, H=32, T=8192, d=128, io="bf16",
                                    q_scale=True, decay_shift=3.0, state_std=0.0, seed=2),
    # Q-Delta: mixed input k + lam_h q, q unscaled
    "qdelta_bf16_b8h8t4096d128": dict(variant="qdelta", B=8, H=8, T=4096, d=128, io="bf16",
                                      q_scale=False, decay_shift=2.0, state_std=0.0, seed=3),
    # Gated DeltaNet-2 at long context
    "gdn2_bf16_b1h32t65536d128": dict(variant="gdn2", B=1, H=32, T=65536, d=128, io="bf16",
                                      q_scale=False, decay_shift=4.0, state_std=0.0, seed=4),
    # the single-token decode step of Gated DeltaNet-2, batch 256 x 32 heads
    "gdn2_decode_b256h32d128": dict(variant="gdn2", B=256, H=32, T=1, d=128, io="bf16",
                                    q_scale=False, decay_shift=4.0, state_std=0.01, seed=5),
}

HEADLINE = "gdn_bf16_b8h16t4096d128"
DECODE = "gdn2_decode_b256h32d128"

# variant -> (decay, erase, write, qmix); mirrors the pages' variant table
KINDS = {
    "deltanet": ("none", "beta", "beta", False),
    "gdn": ("scalar", "beta", "beta", False),
    "kda": ("channel", "beta", "beta", False),
    "qdelta": ("scalar", "beta", "beta", True),
    "gdn2": ("channel", "channel", "channel", False),
}


def config(name: str, **overrides) -> dict:
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    return cfg


def make_inputs(cfg: dict) -> dict:
    """Draw one workload on the CPU.

    ``cfg`` keys: variant, B, H, T, d (or dk, dv), io ("bf16"|"f32"),
    q_scale, decay_shift, state_std, seed, and optional stress knobs:
      decay      override the variant's decay kind ("none"|"scalar"|"channel")
      erase, write  override the gate kinds ("beta"|"channel")
      qmix       override the Q-Delta mix (True|False)
      g_const    use this constant log-decay instead of -softplus(N + c)
      b_scale    erase gate b = b_scale * sigmoid(N)  (e.g. 2 for b in [0, 2])
      lam_const  use this lambda for every head instead of U[0, 1]
      lam_t      draw one lambda per token, [B, T, H] ~ U[0, 1] (time-varying)
      value_beta one beta per value channel, [B, T, H, dv] = sigmoid(N)
                 (erase = write = "value"; replaces beta, b, w)
      epilogue   also draw the output gate [B, T, H, dv] ~ N(0, 1) (I/O
                 dtype) and the RMSNorm weight [dv] = 1 + 0.1 N(0, 1) (fp32)

    Returns a dict of CPU tensors (q, k, v in the I/O dtype; gates and state in
    fp32; unused gates are None) plus the kind fields.
    """
    decay, erase, write, qmix = KINDS[cfg["variant"]]
    decay = cfg.get("decay", decay)
    erase = cfg.get("erase", erase)
    write = cfg.get("write", write)
    if cfg.get("value_beta"):
        erase = write = "value"
    qmix = bool(cfg.get("qmix", qmix))
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    dk = cfg.get("dk", cfg.get("d"))
    dv = cfg.get("dv", cfg.get("d"))
    io = torch.bfloat16 if cfg["io"] == "bf16" else torch.float32
    gen = torch.Generator().manual_seed(int(cfg["seed"]))

    def randn(*shape):
        return torch.randn(*shape, generator=gen, dtype=torch.float32)

    q = randn(B, T, H, dk)
    k = randn(B, T, H, dk)
    v = randn(B, T, H, dv)
    q = q / q.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    if cfg.get("q_scale", False):
        q = q * (1.0 / math.sqrt(dk))

    beta = b = w = None
    if erase == "value":
        beta = torch.sigmoid(randn(B, T, H, dv))
    elif erase == "beta" or write == "beta":
        beta = torch.sigmoid(randn(B, T, H))
    if erase == "channel":
        b = torch.sigmoid(randn(B, T, H, dk)) * float(cfg.get("b_scale", 1.0))
    if write == "channel":
        w = torch.sigmoid(randn(B, T, H, dv))

    g = None
    if decay != "none":
        gshape = (B, T, H) if decay == "scalar" else (B, T, H, dk)
        if "g_const" in cfg:
            g = torch.full(gshape, float(cfg["g_const"]), dtype=torch.float32)
        else:
            g = -torch.nn.functional.softplus(randn(*gshape) + float(cfg["decay_shift"]))

    lam = None
    if qmix:
        if "lam_const" in cfg:
            lam = torch.full((H,), float(cfg["lam_const"]), dtype=torch.float32)
        elif cfg.get("lam_t"):
            lam = torch.rand(B, T, H, generator=gen, dtype=torch.float32)
        else:
            lam = torch.rand(H, generator=gen, dtype=torch.float32)

    std = float(cfg.get("state_std", 0.0))
    state = randn(B, H, dk, dv) * std if std > 0 else None

    out = dict(q=q.to(io).contiguous(), k=k.to(io).contiguous(), v=v.to(io).contiguous(),
               g=g, beta=beta, b=b, w=w, lam=lam, state=state,
               decay=decay, erase=erase, write=write, qmix=qmix)
    if cfg.get("epilogue"):
        out["gate"] = randn(B, T, H, dv).to(io).contiguous()
        out["norm_weight"] = 1.0 + 0.1 * randn(dv)
    return out


def oracle_kwargs(inp: dict) -> dict:
    """The keyword arguments an oracle call takes from ``make_inputs`` output."""
    return dict(decay=inp["decay"], g=inp["g"], erase=inp["erase"], write=inp["write"],
                beta=inp["beta"], b=inp["b"], w=inp["w"], qmix=inp["qmix"], lam=inp["lam"],
                state=inp["state"])


def rel_err(x, ref) -> float:
    """Normative parity metric: max|x - ref| / max|ref| over a whole tensor."""
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(x).max())
    return float(np.abs(x - ref).max() / den)
