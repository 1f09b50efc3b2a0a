"""GPU parity of the HIP chunk kernel and decode step against the float64
oracle, element by element, on seeded inputs small enough for the oracle to
finish in seconds (several 64-token chunks and ragged tails).  Tolerance
metric: max|x - ref| / max|ref| per output tensor (o and the final state),
1e-4 for fp32 I/O and 2e-2 for bf16 I/O.

The stress cases matter: at the workloads' strong decay the chunk's T is tiny
and a kernel with A = I (a broken solve) or without the inter-chunk state
still lands within bf16 tolerance; mild decay and alpha = 1 expose both.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_17_amd as gdr
from synth import config, make_inputs, rel_err
from tests.gpu_util import TOL, assert_parity, run_chunk, run_oracle, say, to_dev, gpu_kwargs

pytestmark = pytest.mark.gpu

H = "gdn_bf16_b8h16t4096d128"
K = "kda_bf16_b4h32t8192d128"
Q = "qdelta_bf16_b8h8t4096d128"
G2 = "gdn2_bf16_b1h32t65536d128"
F = "gdn_f32_b1h2t256d64"

CASES = {
    # the small fp32 workload at full size
    "gdn_f32_full": config(F),
    # each bf16 workload's variant and distributions at a small shape
    "gdn_bf16_small": config(H, B=2, H=2, T=320),
    "kda_bf16_small": config(K, B=1, H=3, T=256),
    "qdelta_bf16_small": config(Q, B=2, H=2, T=256),
    "gdn2_bf16_small": config(G2, B=1, H=2, T=384),
    # stress: mild decay (s1) and alpha = 1 (s2)
    "gdn_mild": config(H, B=1, H=2, T=512, decay_shift=-4.0),
    "deltanet_bf16": config(H, B=1, H=2, T=512, decay="none"),
    "kda_mild": config(K, B=1, H=2, T=512, decay_shift=-4.0),
    "gdn2_mild": config(G2, B=1, H=2, T=512, decay_shift=-4.0),
    # stress: per-channel mild decay at fp32 I/O (s3), at d = 128 (the plain
    # fp32 kernel) and at d = 64 (the fp32 MFMA kernel)
    "kda_f32_mild_d128": config(F, variant="kda", B=1, H=2, T=512, d=128, decay_shift=-4.0),
    "gdn2_f32_mild_d128": config(F, variant="gdn2", B=1, H=2, T=512, d=128, decay_shift=-4.0, state_std=0.1),
    "gdn_f32_mild_d128": config(F, B=1, H=2, T=512, d=128, decay_shift=-4.0, state_std=0.05),
    "qdelta_f32_d128": config(F, variant="qdelta", B=1, H=2, T=320, d=128, q_scale=False, decay_shift=-2.0),
    "deltanet_f32_d128_tail": config(F, B=2, H=1, T=300, d=128, decay="none"),
    "kda_extreme_f32_d128": config(F, variant="kda", B=1, H=2, T=130, d=128, g_const=-20.0),
    "gdn2_f32_d128_dv64": config(F, variant="gdn2", B=1, H=2, T=200, dk=128, dv=64, decay_shift=-4.0),
    "kda_f32_mild": config(F, variant="kda", B=1, H=2, T=512, decay_shift=-4.0),
    "gdn2_f32_mild": config(F, variant="gdn2", B=1, H=2, T=300, decay_shift=-4.0, state_std=0.1),
    "qdelta_f32": config(F, variant="qdelta", B=1, H=2, T=256, q_scale=False),
    "deltanet_f32": config(F, B=1, H=2, T=200, decay="none"),
    # ragged tails (s4) and short sequences
    "gdn_tail300": config(H, B=1, H=2, T=300),
    "gdn2_tail65": config(G2, B=1, H=2, T=65, decay_shift=-4.0),
    "kda_T1": config(K, B=2, H=2, T=1),
    "gdn_T63": config(H, B=1, H=2, T=63, decay_shift=-4.0),
    # extended erase range b in [0, 2] (s5) and lambda = 1 (s6)
    "gdn2_b2": config(G2, B=1, H=2, T=256, decay_shift=-4.0, b_scale=2.0),
    "qdelta_lam1": config(Q, B=1, H=2, T=512, lam_const=1.0, decay_shift=-4.0),
    # extreme decay g = -20 per channel (s7): exercises the exact fallback Gram
    "gdn2_extreme": config(G2, B=1, H=2, T=200, g_const=-20.0),
    "kda_extreme_f32": config(F, variant="kda", B=1, H=2, T=130, g_const=-20.0),
    # the same decay as a scalar: the pipelined kernel, the two-pass scalar
    # form, the plain fp32 two-pass form and the fp32 MFMA kernel
    "gdn_extreme_bf16": config(H, B=1, H=2, T=200, g_const=-20.0),
    "qdelta_extreme_bf16": config(Q, B=1, H=2, T=200, g_const=-20.0),
    "gdn_extreme_f32_d128": config(F, B=1, H=2, T=130, d=128, g_const=-20.0),
    "gdn_extreme_f32": config(F, B=1, H=2, T=130, g_const=-20.0),
    # dk != dv catches transposed operands
    "gdn_dk128_dv64": config(H, B=1, H=2, T=256, dk=128, dv=64, decay_shift=-2.0),
    "kda_dk64_dv128": config(K, B=1, H=2, T=256, dk=64, dv=128, decay_shift=-3.0),
    # dk = dv = 64 on the bf16 kernels, and dv = 256
    "gdn_bf16_d64": config(H, B=1, H=2, T=320, d=64, decay_shift=-3.0),
    "gdn_bf16_d64_wch": config(H, B=2, H=2, T=200, d=64, write="channel", decay_shift=-3.0),
    "gdn_erase_ch_d64": config(H, B=1, H=2, T=200, d=64, erase="channel", decay_shift=-3.0),
    "gdn2_bf16_d64": config(G2, B=1, H=2, T=256, d=64, decay_shift=-4.0),
    "gdn_dv256": config(H, B=1, H=2, T=256, dk=128, dv=256, decay_shift=-3.0),
    "kda_dv256": config(K, B=1, H=2, T=192, dk=128, dv=256, decay_shift=-3.0),
    "gdn2_f32_dv32": config(F, variant="gdn2", B=1, H=2, T=200, dk=64, dv=32, decay_shift=-4.0),
    # gate kinds beyond the variants' own: one gate per key or value channel
    # with the other beta, and the Q-Delta mix, under both decay kinds
    "kda_erase_ch": config(K, B=1, H=2, T=320, erase="channel", decay_shift=-3.0),
    "kda_write_ch": config(K, B=1, H=2, T=200, write="channel", decay_shift=-3.0),
    "kda_qmix": config(K, B=1, H=2, T=256, qmix=True, decay_shift=-3.0),
    "gdn_erase_ch": config(H, B=1, H=2, T=200, erase="channel", decay_shift=-3.0),
    "gdn_write_ch": config(H, B=1, H=2, T=320, write="channel", decay_shift=-3.0),
    # nonzero initial state with per-channel decay
    "kda_state": config(K, B=1, H=2, T=192, decay_shift=-4.0, state_std=0.05),
}


def _two_pass_form(cfg):
    """Shapes that have a two-pass form (taken with a workspace): bf16, dk
    128, few heads (slices of 16 or 32 columns), and either pipelined kernel
    (per-channel decay; or no or a scalar decay with the beta erase gate);
    and every shape of the plain fp32 kernel (fp32 I/O at dk 128)."""
    dk, dv = cfg.get("dk", cfg["d"]), cfg.get("dv", cfg["d"])
    if cfg["io"] == "f32":
        return dk == 128
    decay = cfg.get("decay") or ("channel" if cfg["variant"] in ("kda", "gdn2") else "scalar")
    erase = cfg.get("erase") or ("channel" if cfg["variant"] == "gdn2" else "beta")
    kernel = decay == "channel" or erase == "beta"
    return dk == 128 and kernel and cfg["B"] * cfg["H"] * dv // 64 < 256


# every case as chunk_fwd runs it by default (single pass), and the cases
# with a two-pass form once more in that form
PARITY = [(n, None) for n in sorted(CASES)] + [(n, True) for n in sorted(CASES) if _two_pass_form(CASES[n])]


@pytest.mark.parametrize("name,two_pass", PARITY)
def test_chunk_parity(name, two_pass):
    cfg = CASES[name]
    say(f"[chunk parity] {name} two_pass={two_pass}: {cfg}")
    inp = make_inputs(cfg)
    o, S = run_chunk(inp, two_pass=two_pass)
    o_ref, S_ref = run_oracle(inp)
    assert_parity(name, o, S, o_ref, S_ref, TOL[cfg["io"]])


@pytest.mark.parametrize("name", ["gdn2_bf16_small", "kda_bf16_small", "gdn2_extreme", "gdn_bf16_small",
                                  "qdelta_lam1", "deltanet_bf16"])
def test_two_pass_form(name):
    """The two-pass form is what the plan reports with a workspace, and its
    16- and 32-column slices give bitwise-identical results."""
    cfg = CASES[name]
    inp = make_inputs(cfg)
    d = to_dev(inp)
    ws = gdr.new_workspace(d["q"], d["k"], d["v"], **gpu_kwargs(d))
    assert ws is not None
    assert gdr.plan(d["q"], d["k"], d["v"], workspace=ws, **gpu_kwargs(d))["passes"] == 2
    assert gdr.plan(d["q"], d["k"], d["v"], **gpu_kwargs(d))["passes"] == 1
    outs = []
    for wdt in (16, 32):
        say(f"[two-pass] {name} dv_split={wdt}")
        outs.append(run_chunk(inp, dv_split=wdt, two_pass=True))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("name", ["gdn_bf16_small", "gdn2_bf16_small", "kda_f32_mild", "kda_f32_mild_d128"])
def test_slice_width_does_not_change_results(name):
    """Every value-slice width gives bitwise-identical results (the per-column
    arithmetic does not depend on how columns are split over workgroups)."""
    cfg = CASES[name]
    inp = make_inputs(cfg)
    widths = (16, 32) if cfg["io"] == "f32" else (16, 32, 64)
    if cfg["io"] == "f32" and cfg.get("d") == 128:
        widths = (16, 0)   # the plain kernel's one width, chosen or given
    ref = None
    for wdt in widths:
        say(f"[slice] {name} dv_split={wdt}")
        o, S = run_chunk(inp, dv_split=wdt, two_pass=False)
        if ref is None:
            ref = (o, S)
        else:
            assert np.array_equal(o, ref[0]) and np.array_equal(S, ref[1]), f"dv_split={wdt} differs"


def test_deterministic():
    inp = make_inputs(CASES["kda_bf16_small"])
    say("[determinism] kda_bf16_small x2")
    a = run_chunk(inp)
    b = run_chunk(inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("name", ["gdn_bf16_small", "gdn2_mild", "gdn_f32_full"])
def test_streaming_handoff(name):
    """One call over T tokens equals two calls over T/2 with the final state
    handed over (the split is on a chunk boundary, so bitwise equal)."""
    cfg = dict(CASES[name])
    cfg["T"] = 256
    inp = make_inputs(cfg)
    d = to_dev(inp)
    say(f"[streaming] {name}")
    o, S = gdr.chunk_fwd(d["q"], d["k"], d["v"], **gpu_kwargs(d))
    half = {}
    for key, val in d.items():
        if isinstance(val, torch.Tensor) and key not in ("lam", "state"):
            half[key] = (val[:, :128].contiguous(), val[:, 128:].contiguous())
    kw1 = gpu_kwargs(d)
    kw2 = gpu_kwargs(d)
    for key in ("g", "beta", "b", "w"):
        if d[key] is not None:
            kw1[key], kw2[key] = half[key]
    o1, S1 = gdr.chunk_fwd(half["q"][0], half["k"][0], half["v"][0], **kw1)
    kw2["state"] = S1
    o2, S2 = gdr.chunk_fwd(half["q"][1], half["k"][1], half["v"][1], **kw2)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], dim=1), o)
    assert torch.equal(S2, S)


def test_zero_length_copies_state():
    inp = make_inputs(config(H, B=1, H=2, T=64))
    d = to_dev(inp)
    say("[T=0]")
    q0 = d["q"][:, :0].contiguous()
    o, S = gdr.chunk_fwd(q0, q0, d["v"][:, :0].contiguous(), g=d["g"][:, :0].contiguous(),
                         beta=d["beta"][:, :0].contiguous(), state=d["state"])
    torch.cuda.synchronize()
    assert o.shape[1] == 0 and torch.equal(S, d["state"])
    o, S = gdr.chunk_fwd(q0, q0, d["v"][:, :0].contiguous(), g=d["g"][:, :0].contiguous(),
                         beta=d["beta"][:, :0].contiguous())
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0


def test_state_in_place():
    inp = make_inputs(config(K, B=1, H=2, T=128, state_std=0.05))
    d = to_dev(inp)
    say("[state in place]")
    o_ref, S_ref = gdr.chunk_fwd(d["q"], d["k"], d["v"], **gpu_kwargs(d))
    st = d["state"].clone()
    kw = gpu_kwargs(d)
    kw["state"] = st
    o, S = gdr.chunk_fwd(d["q"], d["k"], d["v"], state_out=st, **kw)
    torch.cuda.synchronize()
    assert S.data_ptr() == st.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


# ---------------------------------------------------------------------------
# decode step

STEP_CASES = {
    "gdn2_decode_small": config("gdn2_decode_b256h32d128", B=4, H=4),
    "gdn_step_f32": config(F, T=1, B=3, H=2, state_std=0.1),
    "kda_step": config(K, T=1, B=2, H=3, state_std=0.1),
    "qdelta_step": config(Q, T=1, B=2, H=3, state_std=0.1),
    "deltanet_step_dk64_dv128": config(H, T=1, B=2, H=2, dk=64, dv=128, decay="none", state_std=0.1),
}


@pytest.mark.parametrize("name", sorted(STEP_CASES))
def test_step_parity(name):
    cfg = STEP_CASES[name]
    say(f"[step parity] {name}")
    inp = make_inputs(cfg)
    d = to_dev(inp)
    o, S = gdr.recurrent_step(d["q"], d["k"], d["v"], **gpu_kwargs(d))
    torch.cuda.synchronize()
    o_ref, S_ref = run_oracle(inp)
    assert_parity(name, o.float().cpu().numpy(), S.cpu().numpy(), o_ref, S_ref, TOL[cfg["io"]])


def test_step_matches_chunk_over_a_sequence():
    """T decode steps with the state handed over equal one chunked call."""
    cfg = config(G2, B=1, H=2, T=70, decay_shift=-4.0, state_std=0.05)
    inp = make_inputs(cfg)
    d = to_dev(inp)
    say("[step vs chunk]")
    o_c, S_c = gdr.chunk_fwd(d["q"], d["k"], d["v"], **gpu_kwargs(d))
    st = d["state"].clone()
    outs = []
    for t in range(cfg["T"]):
        kw = gpu_kwargs(d)
        for key in ("g", "beta", "b", "w"):
            if d[key] is not None:
                kw[key] = d[key][:, t:t + 1].contiguous()
        kw["state"] = st
        o_t, _ = gdr.recurrent_step(d["q"][:, t:t + 1].contiguous(), d["k"][:, t:t + 1].contiguous(),
                                    d["v"][:, t:t + 1].contiguous(), state_out=st, **kw)
        outs.append(o_t)
    torch.cuda.synchronize()
    o_s = torch.cat(outs, dim=1).float()
    assert rel_err(o_s.cpu().numpy(), o_c.float().cpu().numpy()) <= TOL["bf16"]
    assert rel_err(st.cpu().numpy(), S_c.cpu().numpy()) <= TOL["bf16"]


def test_step_qdelta_contraction_on_gpu():
    """Lemma 3.1 of the Q-Delta page at alpha = 1: the mixed prediction error
    along x = k + lam q shrinks by exactly |1 - beta k.x| in one step."""
    cfg = config(Q, T=1, B=4, H=4, state_std=0.3, decay="none")
    inp = make_inputs(cfg)
    d = to_dev(inp)
    say("[step contraction]")
    fq = torch.float32
    d["q"], d["k"], d["v"] = d["q"].to(fq), d["k"].to(fq), d["v"].to(fq)
    o, S1 = gdr.recurrent_step(d["q"], d["k"], d["v"], **gpu_kwargs(d))
    torch.cuda.synchronize()
    q, k, v = (inp[x].double()[:, 0] for x in ("q", "k", "v"))  # [B,H,d]
    lam = inp["lam"].double()[None, :, None]
    x = k + lam * q
    beta = inp["beta"].double()[:, 0]
    a = (k * x).sum(-1)
    S0 = inp["state"].double()
    before = (v - torch.einsum("bhcv,bhc->bhv", S0, x)).norm(dim=-1)
    after = (v - torch.einsum("bhcv,bhc->bhv", S1.cpu().double(), x)).norm(dim=-1)
    expect = (1 - beta * a).abs() * before
    assert torch.allclose(after, expect, rtol=1e-4, atol=1e-5)


def _yu_chunk_form(inp):
    """The chunk WY form with Y = A E_bar and U = A Z ([GDN2] key design 2), in
    float64 through the oracle's literal mirror, on every (b, h)."""
    from oracle.chunk_mirror import chunk_forward_one
    q, k, v = (inp[x].double().numpy() for x in ("q", "k", "v"))
    B, T, H, dk = k.shape
    dv = v.shape[3]
    beta = inp["beta"].double().numpy()
    g = inp["g"].double().numpy() if inp["g"] is not None else np.zeros((B, T, H))
    lam = inp["lam"].double().numpy() if inp["lam"] is not None else np.zeros(H)
    S0 = inp["state"].double().numpy() if inp["state"] is not None else np.zeros((B, H, dk, dv))
    o = np.zeros((B, T, H, dv))
    S = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            x = k[b, :, h] + (lam[h] * q[b, :, h] if inp["qmix"] else 0.0)
            e = beta[b, :, h, None] * x
            z = beta[b, :, h, None] * v[b, :, h]
            gg = np.repeat(g[b, :, h, None], dk, axis=1)
            o[b, :, h], S[b, h] = chunk_forward_one(q[b, :, h], k[b, :, h], e, z, gg, S0[b, h])
    return o, S


@pytest.mark.parametrize("name", ["gdn_bf16_small", "qdelta_bf16_small", "deltanet_bf16", "gdn_tail300"])
def test_pipelined_kernel_matches_the_yu_chunk_form(name):
    """The pipelined kernel evaluates W = A (Z - E_bar S) instead of the page's
    U - Y S; checked here directly against the Y / U form."""
    cfg = CASES[name]
    inp = make_inputs(cfg)
    assert inp["decay"] != "channel" and inp["erase"] == "beta" and cfg["io"] == "bf16"
    o_ref, S_ref = _yu_chunk_form(inp)
    for two_pass in (False, True):
        say(f"[Y/U form] {name} two_pass={two_pass}")
        o, S = run_chunk(inp, two_pass=two_pass)
        assert_parity(name, o, S, o_ref, S_ref, TOL[cfg["io"]])
