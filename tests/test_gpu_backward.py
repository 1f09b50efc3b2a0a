"""GPU parity of the backward (gdr_chunk_bwd) against the float64 oracle's
adjoint (``oracle.backward``, pinned by finite differences): every gradient
of every input, element by element, max|x - ref| / max|ref| per tensor, at
the forward's bars (1e-4 for fp32 I/O, 2e-2 for bf16 I/O; the backward
accumulates in fp32, its record recurrence and reverse state pass multiply
in split precision, about 16 bits per operand, so both land far below them).  The cases
cover each variant and gate kind, the mild-decay and alpha = 1 stress cases,
extreme decay, ragged and single-chunk lengths, dk != dv and T = 0."""

import numpy as np
import pytest
import torch

import gated_delta_rule_17_amd as gdr
from oracle import gdr_recurrence_vjp
from synth import config, make_inputs, oracle_kwargs, rel_err
from tests.gpu_util import TOL, gpu_kwargs, say, to_dev

pytestmark = pytest.mark.gpu

H = "gdn_bf16_b8h16t4096d128"
K = "kda_bf16_b4h32t8192d128"
Q = "qdelta_bf16_b8h8t4096d128"
G2 = "gdn2_bf16_b1h32t65536d128"
F = "gdn_f32_b1h2t256d64"

CASES = {
    "gdn_bf16_mild": config(H, B=2, H=2, T=200, decay_shift=-4.0, state_std=0.05),
    "deltanet_bf16": config(H, B=1, H=2, T=192, decay="none"),
    "kda_bf16_mild": config(K, B=1, H=2, T=150, decay_shift=-4.0),
    "gdn2_bf16_mild": config(G2, B=1, H=2, T=130, decay_shift=-4.0, state_std=0.05),
    "gdn2_bf16_strong": config(G2, B=1, H=2, T=128),
    "qdelta_bf16": config(Q, B=2, H=2, T=100, decay_shift=-3.0),
    "qdelta_lam_t_f32": config(F, variant="qdelta", B=1, H=2, T=90, d=128, lam_t=True, q_scale=False),
    "gdn_f32_d64": config(F, B=2, H=2, T=160, state_std=0.1),
    "gdn2_f32_dk64_dv128": config(F, variant="gdn2", B=1, H=2, T=70, dk=64, dv=128, decay_shift=-4.0),
    "kda_f32_dk128_dv64": config(F, variant="kda", B=1, H=2, T=64, dk=128, dv=64, decay_shift=-4.0),
    "gdn2_extreme": config(G2, B=1, H=2, T=100, g_const=-20.0),
    "gdn_bf16_extreme": config(H, B=1, H=2, T=100, g_const=-20.0),
    # bf16 at dk 64 (the exact prep and the product and key pass at 64 key
    # channels) and dv 64 (one 64-column slice)
    "gdn_bf16_d64": config(H, B=1, H=2, T=150, d=64, decay_shift=-3.0),
    "qdelta_bf16_dk64_dv128": config(Q, B=1, H=2, T=130, dk=64, dv=128, decay_shift=-3.0),
    "gdn_bf16_dk128_dv64": config(H, B=2, H=1, T=100, dk=128, dv=64, decay_shift=-2.0),
    "gdn_erase_ch_f32": config(F, B=1, H=2, T=80, erase="channel", decay_shift=-3.0),
    # bf16 under a scalar decay: the record recurrence and the state pass form
    # the factor rows from the inputs (per-channel erase gate; lambda per token)
    "gdn_erase_ch_bf16": config(H, B=1, H=2, T=80, erase="channel", decay_shift=-3.0),
    "qdelta_lam_t_bf16": config(Q, B=1, H=2, T=90, lam_t=True, decay_shift=-3.0),
    "kda_write_ch_bf16": config(K, B=1, H=2, T=96, write="channel", decay_shift=-3.0),
    "gdn2_T1": config(G2, B=2, H=2, T=1, state_std=0.1),
}

GRAD_OF = {"dq": "q", "dk": "k", "dv": "v", "dg": "g", "dbeta": "beta", "db": "b", "dw": "w", "dlam": "lam"}


def _cotangents(inp, seed):
    gen = torch.Generator().manual_seed(1000 + seed)
    do = torch.randn(inp["v"].shape, generator=gen).to(inp["q"].dtype)
    B, H, dk, dv = inp["q"].shape[0], inp["q"].shape[2], inp["q"].shape[3], inp["v"].shape[3]
    dS = torch.randn(B, H, dk, dv, generator=gen) * 0.1
    return do, dS


def _check(name, inp, got, ref, tol):
    worst = 0.0
    for key in ("dq", "dk", "dv", "dg", "dbeta", "db", "dw", "dlam", "dstate"):
        r = ref.get(key)
        if r is None:
            continue
        x = got[key].cpu().numpy()
        assert x.shape == r.shape, (key, x.shape, r.shape)
        assert np.isfinite(x).all(), f"{name}: non-finite {key}"
        e = rel_err(x, r)
        worst = max(worst, e)
        say(f"    {name} {key}: rel err {e:.3e}")
        assert e <= tol, f"{name}: {key} {e:.3e} > {tol:.0e}"
    return worst


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_parity(name):
    cfg = CASES[name]
    say(f"[backward] {name}: {cfg}")
    inp = make_inputs(cfg)
    do, dS = _cotangents(inp, len(name))
    d = to_dev(inp)
    ws = gdr.bwd_workspace_size(d["q"], d["k"], d["v"], do.cuda(), **gpu_kwargs(d))
    say(f"    workspace {ws} bytes")
    got = gdr.chunk_bwd(d["q"], d["k"], d["v"], do.cuda(), dstate=dS.cuda(), **gpu_kwargs(d))
    torch.cuda.synchronize()
    ref = gdr_recurrence_vjp(inp["q"], inp["k"], inp["v"], do, dstate=dS, **oracle_kwargs(inp))
    _check(name, inp, got, ref, TOL[cfg["io"]])


def test_backward_is_deterministic_and_needs_no_final_cotangent():
    cfg = CASES["gdn2_bf16_mild"]
    inp = make_inputs(cfg)
    do, _ = _cotangents(inp, 3)
    d = to_dev(inp)
    say("[backward] repeat, no dstate")
    a = gdr.chunk_bwd(d["q"], d["k"], d["v"], do.cuda(), **gpu_kwargs(d))
    b = gdr.chunk_bwd(d["q"], d["k"], d["v"], do.cuda(), **gpu_kwargs(d))
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
    ref = gdr_recurrence_vjp(inp["q"], inp["k"], inp["v"], do, **oracle_kwargs(inp))
    _check("no dstate", inp, a, ref, TOL[cfg["io"]])


def test_backward_zero_length():
    cfg = config(H, B=1, H=2, T=64, state_std=0.05)
    inp = make_inputs(cfg)
    d = to_dev(inp)
    z = lambda x: x[:, :0].contiguous()  # noqa: E731
    dS = torch.randn(1, 2, 128, 128, device="cuda")
    say("[backward] T = 0")
    got = gdr.chunk_bwd(z(d["q"]), z(d["k"]), z(d["v"]), z(d["v"]), g=z(d["g"]), beta=z(d["beta"]),
                        state=d["state"], dstate=dS)
    torch.cuda.synchronize()
    assert torch.equal(got["dstate"], dS)
