"""GPU parity of the variants beyond the five workloads' own, of the fully
recurrent form and of the output epilogue, each against the float64 oracle
(max|x - ref| / max|ref| per tensor; 1e-4 for fp32 I/O, 2e-2 for bf16 I/O):

* time-varying lambda_t (Q-Delta page, key design 2) and one beta per value
  channel ("Chapter 11", 11.3) through gdr_chunk_fwd and gdr_recurrent_step;
* gdr_recurrent_fwd, the token loop in one kernel (Q-Delta page, key design
  3), for every variant and gate kind at short and ragged T;
* the RMSNorm + SiLU output epilogue ("Chapter 11", 11.3), standalone and
  fused into the recurrent kernels and after the chunk kernels.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_17_amd as gdr
from oracle import output_norm_gate as oracle_norm_gate
from synth import config, make_inputs, rel_err
from tests.gpu_util import TOL, assert_parity, gpu_kwargs, run_oracle, say, to_dev

pytestmark = pytest.mark.gpu

H = "gdn_bf16_b8h16t4096d128"
K = "kda_bf16_b4h32t8192d128"
Q = "qdelta_bf16_b8h8t4096d128"
G2 = "gdn2_bf16_b1h32t65536d128"
F = "gdn_f32_b1h2t256d64"

# ---- chunk form: lambda_t and the per-value-channel beta ------------------

VARIANT_CASES = {
    "qdelta_lam_t_bf16": config(Q, B=2, H=2, T=320, lam_t=True, decay_shift=-3.0),
    "qdelta_lam_t_f32_d128": config(F, variant="qdelta", B=1, H=2, T=300, d=128, lam_t=True, q_scale=False),
    "qdelta_lam_t_f32_d64": config(F, variant="qdelta", B=1, H=3, T=200, lam_t=True, q_scale=False,
                                   decay_shift=-4.0),
    "gdn_value_beta_bf16": config(H, B=1, H=2, T=384, value_beta=True, decay_shift=-3.0),
    "gdn_value_beta_f32": config(F, B=1, H=2, T=256, d=128, value_beta=True, decay_shift=-4.0, state_std=0.1),
    "kda_value_beta_bf16": config(K, B=1, H=2, T=256, value_beta=True, decay_shift=-4.0),
    "deltanet_value_beta_f32_dk64_dv128": config(F, B=1, H=2, T=200, dk=64, dv=128, decay="none",
                                                 value_beta=True),
    "gdn2_lam_t_kda_mix": config(K, B=1, H=2, T=192, qmix=True, lam_t=True, decay_shift=-4.0),
}


@pytest.mark.parametrize("two_pass", [False, True])
@pytest.mark.parametrize("name", sorted(VARIANT_CASES))
def test_variant_chunk_parity(name, two_pass):
    """Through the plain kernel's single pass and its two-pass form."""
    cfg = VARIANT_CASES[name]
    say(f"[variant chunk] {name} two_pass={two_pass}: {cfg}")
    inp = make_inputs(cfg)
    d = to_dev(inp)
    o, S = gdr.chunk_fwd(d["q"], d["k"], d["v"], two_pass=two_pass, **gpu_kwargs(d))
    torch.cuda.synchronize()
    o_ref, S_ref = run_oracle(inp)
    assert_parity(name, o.float().cpu().numpy(), S.cpu().numpy(), o_ref, S_ref, TOL[cfg["io"]])


@pytest.mark.parametrize("name", ["qdelta_lam_t_bf16", "gdn_value_beta_f32", "kda_value_beta_bf16"])
def test_variant_step_parity(name):
    cfg = dict(VARIANT_CASES[name], T=1, state_std=0.1)
    say(f"[variant step] {name}")
    inp = make_inputs(cfg)
    d = to_dev(inp)
    o, S = gdr.recurrent_step(d["q"], d["k"], d["v"], **gpu_kwargs(d))
    torch.cuda.synchronize()
    o_ref, S_ref = run_oracle(inp)
    assert_parity(name, o.float().cpu().numpy(), S.cpu().numpy(), o_ref, S_ref, TOL[cfg["io"]])


# ---- the recurrent form ------------------------------------------------------

RECUR_CASES = {
    "gdn_bf16_T16": config(H, B=4, H=4, T=16, state_std=0.05),
    "gdn_bf16_T64": config(H, B=2, H=4, T=64, decay_shift=-4.0),
    "kda_bf16_T37": config(K, B=2, H=3, T=37, decay_shift=-4.0, state_std=0.05),
    "qdelta_bf16_T64": config(Q, B=2, H=2, T=64, lam_const=1.0, decay_shift=-4.0),
    "qdelta_lam_t_bf16_T50": config(Q, B=2, H=2, T=50, lam_t=True),
    "gdn2_bf16_T100": config(G2, B=1, H=4, T=100, decay_shift=-4.0),
    "gdn2_b2_T16": config(G2, B=2, H=2, T=16, b_scale=2.0),
    "deltanet_bf16_T80": config(H, B=1, H=2, T=80, decay="none"),
    "value_beta_bf16_T33": config(H, B=2, H=2, T=33, value_beta=True, decay_shift=-3.0),
    "gdn_f32_T64": config(F, B=2, H=2, T=64, state_std=0.1),
    "kda_f32_d128_T20": config(F, variant="kda", B=1, H=2, T=20, d=128, decay_shift=-4.0),
    "gdn2_f32_dk64_dv128_T40": config(F, variant="gdn2", B=1, H=2, T=40, dk=64, dv=128, decay_shift=-4.0),
    "gdn_bf16_dk128_dv64_T24": config(H, B=2, H=2, T=24, dk=128, dv=64),
    "gdn2_extreme_T30": config(G2, B=1, H=2, T=30, g_const=-20.0),
    "kda_T1": config(K, B=3, H=2, T=1, state_std=0.1),
}


@pytest.mark.parametrize("name", sorted(RECUR_CASES))
def test_recurrent_parity(name):
    cfg = RECUR_CASES[name]
    say(f"[recurrent] {name}: {cfg}")
    inp = make_inputs(cfg)
    d = to_dev(inp)
    o, S = gdr.recurrent_fwd(d["q"], d["k"], d["v"], **gpu_kwargs(d))
    torch.cuda.synchronize()
    o_ref, S_ref = run_oracle(inp)
    assert_parity(name, o.float().cpu().numpy(), S.cpu().numpy(), o_ref, S_ref, TOL[cfg["io"]])


def test_recurrent_streaming_handoff():
    """Two calls with the state handed over agree with one call, at a split
    that is not a multiple of the 8-token staging block.  The kernel folds
    each channel's running decay into the state at the end of a call (and
    only when needed inside one), so a split moves roundings: the fp32 state
    agrees to a few fp32 roundings and the bf16 output to its own rounding
    (one bf16 step is 2^-8 of the value)."""
    cfg = config(G2, B=2, H=2, T=45, decay_shift=-4.0, state_std=0.05)
    inp = make_inputs(cfg)
    d = to_dev(inp)
    say("[recurrent streaming]")
    o, S = gdr.recurrent_fwd(d["q"], d["k"], d["v"], **gpu_kwargs(d))
    cut = 19
    kw1, kw2 = gpu_kwargs(d), gpu_kwargs(d)
    for key in ("g", "beta", "b", "w"):
        if d[key] is not None:
            kw1[key], kw2[key] = d[key][:, :cut].contiguous(), d[key][:, cut:].contiguous()
    sl = lambda x, a, b: x[:, a:b].contiguous()  # noqa: E731
    o1, S1 = gdr.recurrent_fwd(sl(d["q"], 0, cut), sl(d["k"], 0, cut), sl(d["v"], 0, cut), **kw1)
    kw2["state"] = S1
    o2, S2 = gdr.recurrent_fwd(sl(d["q"], cut, 45), sl(d["k"], cut, 45), sl(d["v"], cut, 45), **kw2)
    torch.cuda.synchronize()
    o_split = torch.cat([o1, o2], dim=1).float().cpu().numpy()
    assert rel_err(o_split, o.float().cpu().numpy()) <= 2.0 ** -8
    assert rel_err(S2.cpu().numpy(), S.cpu().numpy()) <= 1e-5


def test_recurrent_matches_the_chunk_form():
    cfg = config(K, B=2, H=2, T=96, decay_shift=-4.0, state_std=0.05)
    inp = make_inputs(cfg)
    d = to_dev(inp)
    say("[recurrent vs chunk]")
    o_r, S_r = gdr.recurrent_fwd(d["q"], d["k"], d["v"], **gpu_kwargs(d))
    o_c, S_c = gdr.chunk_fwd(d["q"], d["k"], d["v"], **gpu_kwargs(d))
    torch.cuda.synchronize()
    assert rel_err(o_r.float().cpu().numpy(), o_c.float().cpu().numpy()) <= TOL["bf16"]
    assert rel_err(S_r.cpu().numpy(), S_c.cpu().numpy()) <= TOL["bf16"]


def test_recurrent_state_in_place_and_zero_length():
    cfg = config(H, B=2, H=2, T=20, state_std=0.05)
    inp = make_inputs(cfg)
    d = to_dev(inp)
    say("[recurrent in place / T=0]")
    o_ref, S_ref = gdr.recurrent_fwd(d["q"], d["k"], d["v"], **gpu_kwargs(d))
    st = d["state"].clone()
    kw = gpu_kwargs(d)
    kw["state"] = st
    o, S = gdr.recurrent_fwd(d["q"], d["k"], d["v"], state_out=st, **kw)
    q0 = d["q"][:, :0].contiguous()
    o0, S0 = gdr.recurrent_fwd(q0, q0, d["v"][:, :0].contiguous(), g=d["g"][:, :0].contiguous(),
                               beta=d["beta"][:, :0].contiguous(), state=d["state"])
    torch.cuda.synchronize()
    assert S.data_ptr() == st.data_ptr() and torch.equal(o, o_ref) and torch.equal(S, S_ref)
    assert o0.shape[1] == 0 and torch.equal(S0, d["state"])


# ---- the output epilogue -----------------------------------------------------

def _epilogue_ref(inp, o_ref):
    return oracle_norm_gate(o_ref, inp["gate"], inp["norm_weight"])


@pytest.mark.parametrize("io,dv", [("bf16", 128), ("bf16", 64), ("f32", 128), ("bf16", 256), ("f32", 64)])
def test_epilogue_standalone(io, dv):
    gen = torch.Generator().manual_seed(dv)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    o = (torch.randn(3, 37, 5, dv, generator=gen) * 0.3).to(dt)
    gate = torch.randn(3, 37, 5, dv, generator=gen).to(dt)
    wt = 1.0 + 0.1 * torch.randn(dv, generator=gen)
    say(f"[epilogue] io={io} dv={dv}")
    y = gdr.output_norm_gate(o.cuda(), gate.cuda(), wt.cuda())
    y_in_place = o.cuda()
    gdr.output_norm_gate(y_in_place, gate.cuda(), wt.cuda(), out=y_in_place)
    torch.cuda.synchronize()
    ref = oracle_norm_gate(o, gate, wt)
    err = rel_err(y.float().cpu().numpy(), ref)
    say(f"    rel err {err:.3e}")
    assert err <= TOL[io]
    assert torch.equal(y, y_in_place)


@pytest.mark.parametrize("entry", ["chunk", "recurrent", "step"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_epilogue_fused(entry, io):
    base = config(G2, B=2, H=2, T=1 if entry == "step" else 70, decay_shift=-4.0, state_std=0.05,
                  epilogue=True)
    if io == "f32":
        base.update(io="f32", d=64)
    inp = make_inputs(base)
    d = to_dev(inp)
    say(f"[epilogue fused] {entry} io={io}")
    fn = {"chunk": gdr.chunk_fwd, "recurrent": gdr.recurrent_fwd, "step": gdr.recurrent_step}[entry]
    y, S = fn(d["q"], d["k"], d["v"], gate=d["gate"], norm_weight=d["norm_weight"], **gpu_kwargs(d))
    torch.cuda.synchronize()
    o_ref, S_ref = run_oracle(inp)
    y_ref = _epilogue_ref(inp, o_ref)
    assert_parity(f"epilogue {entry} {io}", y.float().cpu().numpy(), S.cpu().numpy(), y_ref, S_ref, TOL[io])


# ---- the plain fp32 kernel's two recurrences ----------------------------------

@pytest.mark.parametrize("name,cfg", [
    ("gdn_f32_d128", config(F, B=2, H=2, T=300, d=128, decay_shift=-3.0, state_std=0.1)),
    ("kda_f32_d128_dv64", config(F, variant="kda", B=1, H=3, T=200, dk=128, dv=64, decay_shift=-4.0)),
    ("kda_bf16_lam_t", config(K, B=1, H=2, T=150, qmix=True, lam_t=True, decay_shift=-4.0)),
    # bf16 under a scalar decay: the matrix-core recurrence forms the factor rows
    ("qdelta_bf16_lam_t", config(Q, B=1, H=2, T=150, lam_t=True, decay_shift=-4.0)),
    ("gdn2_bf16_value_beta", config(G2, B=1, H=2, T=150, value_beta=True, decay_shift=-4.0)),
])
def test_plain_two_pass_recurrences(name, cfg):
    """The two-pass plain form's recurrence on the matrix cores (64-column
    slices) and on the vector ALUs (a 16-column split, or the per-value-channel
    beta's substitution), and the single pass, each against the oracle."""
    inp = make_inputs(cfg)
    d = to_dev(inp)
    o_ref, S_ref = run_oracle(inp)
    for two_pass, split in ((True, 0), (True, 16), (False, 0)):
        say(f"[plain recurrences] {name} two_pass={two_pass} dv_split={split}")
        plan = gdr.plan(d["q"], d["k"], d["v"], dv_split=split, workspace=gdr.new_workspace(
            d["q"], d["k"], d["v"], **gpu_kwargs(d)) if two_pass else None, **gpu_kwargs(d))
        assert plan["passes"] == (2 if two_pass else 1)
        # (the per-value-channel beta keeps 16-column slices: per-column systems)
        assert plan["dv_slice"] == (64 if two_pass and not split and not cfg.get("value_beta") else 16)
        o, S = gdr.chunk_fwd(d["q"], d["k"], d["v"], dv_split=split, two_pass=two_pass, **gpu_kwargs(d))
        torch.cuda.synchronize()
        assert_parity(f"{name} {two_pass} {split}", o.float().cpu().numpy(), S.cpu().numpy(), o_ref, S_ref,
                      TOL[cfg["io"]])
