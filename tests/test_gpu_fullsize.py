"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times: the whole batch runs on the GPU, and sampled (batch, head)
sequences (every token of each) are compared with the float64 oracle, which
is run on just those sequences."""

import numpy as np
import pytest
import torch

import gated_delta_rule_17_amd as gdr
from synth import CONFIGS, DECODE, config, make_inputs
from tests.gpu_util import TOL, assert_parity, elementwise_rel, gpu_kwargs, run_oracle, say, to_dev

pytestmark = pytest.mark.gpu

FULL = ["gdn_bf16_b8h16t4096d128", "kda_bf16_b4h32t8192d128", "qdelta_bf16_b8h8t4096d128",
        "gdn2_bf16_b1h32t65536d128", "gdn_f32_b8h16t4096d128"]


def _config(name):
    # fp32 I/O at d = 128 on the headline's shape (the plain kernel; its
    # two-pass form is what the benchmark times)
    if name == "gdn_f32_b8h16t4096d128":
        return config("gdn_bf16_b8h16t4096d128", io="f32")
    return config(name)


def _sample_heads(B, H, n, seed):
    rng = np.random.default_rng(seed)
    pairs = {(0, 0), (B - 1, H - 1)}
    while len(pairs) < n:
        pairs.add((int(rng.integers(B)), int(rng.integers(H))))
    return sorted(pairs)


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_heads(name):
    cfg = _config(name)
    say(f"[full] {name}: generating")
    inp = make_inputs(cfg)
    d = to_dev(inp)
    # the form bench.py times (two passes where the library offers them), and
    # the single pass too where that differs
    forms = [None] + ([False] if gdr.workspace_size(d["q"], d["k"], d["v"], **gpu_kwargs(d)) else [])
    results = []
    for two_pass in forms:
        ws = None if two_pass is False else gdr.new_workspace(d["q"], d["k"], d["v"], **gpu_kwargs(d))
        plan = gdr.plan(d["q"], d["k"], d["v"], workspace=ws, **gpu_kwargs(d))
        say(f"[full] {name}: chunk_fwd two_pass={two_pass} {plan}")
        o, S = gdr.chunk_fwd(d["q"], d["k"], d["v"], two_pass=two_pass, workspace=ws, **gpu_kwargs(d))
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
        results.append((two_pass, o.float().cpu(), S.cpu()))
        del o, S, ws
    heads = _sample_heads(cfg["B"], cfg["H"], 4 if cfg["T"] > 10000 else 8, seed=len(name))
    say(f"[full] {name}: oracle on heads {heads}")
    o_ref, S_ref = run_oracle(inp, heads)
    for two_pass, o, S in results:
        worst = (0.0, None)
        for (b, h), orf, srf in zip(heads, o_ref, S_ref):
            eo, es = assert_parity(f"{name} two_pass={two_pass} b={b} h={h}", o[b, :, h].numpy(),
                                   S[b, h].numpy(), orf, srf, TOL[cfg["io"]])
            worst = max(worst, (max(eo, es), (b, h)))
            say(f"      elementwise |d|/(|ref|+1e-6): o {elementwise_rel(o[b, :, h].numpy(), orf):.2e} "
                f"S {elementwise_rel(S[b, h].numpy(), srf):.2e}")
        say(f"    {name} two_pass={two_pass}: worst (b, h) slice {worst[1]} at {worst[0]:.3e}")
    del d, results
    torch.cuda.empty_cache()


def test_full_size_decode_step():
    cfg = config(DECODE)
    say(f"[full] {DECODE}")
    inp = make_inputs(cfg)
    d = to_dev(inp)
    o, S = gdr.recurrent_step(d["q"], d["k"], d["v"], **gpu_kwargs(d))
    torch.cuda.synchronize()
    heads = _sample_heads(cfg["B"], cfg["H"], 64, seed=5)
    o_ref, S_ref = run_oracle(inp, heads)
    for (b, h), orf, srf in zip(heads, o_ref, S_ref):
        assert_parity(f"decode b={b} h={h}", o[b, :, h].float().cpu().numpy(), S[b, h].cpu().numpy(),
                      orf, srf, TOL[cfg["io"]])


def test_full_size_backward_sampled_heads():
    """The backward of the headline workload at its full size (B8 H16
    T4096): every gradient of three sampled heads against the float64
    adjoint run on just those heads."""
    from oracle import gdr_recurrence_vjp
    from synth import oracle_kwargs, rel_err

    cfg = config("gdn_bf16_b8h16t4096d128")
    say("[full bwd] generating")
    inp = make_inputs(cfg)
    d = to_dev(inp)
    gen = torch.Generator().manual_seed(77)
    do = torch.randn(inp["v"].shape, generator=gen).to(inp["q"].dtype)
    dS = torch.randn(inp["state"].shape, generator=gen) * 0.1
    got = gdr.chunk_bwd(d["q"], d["k"], d["v"], do.cuda(), dstate=dS.cuda(), **gpu_kwargs(d))
    torch.cuda.synchronize()
    for key, val in got.items():
        assert torch.isfinite(val).all(), key
    for b, h in _sample_heads(cfg["B"], cfg["H"], 3, seed=11):
        say(f"[full bwd] oracle adjoint of b={b} h={h}")
        tok = lambda x: x[b:b + 1, :, h:h + 1].contiguous()  # noqa: E731
        sub = {key: (tok(val) if isinstance(val, torch.Tensor) and val.dim() >= 3 and key != "state" else val)
               for key, val in inp.items()}
        sub["state"] = inp["state"][b:b + 1, h:h + 1].contiguous()
        ref = gdr_recurrence_vjp(sub["q"], sub["k"], sub["v"], tok(do),
                                 dstate=dS[b:b + 1, h:h + 1].contiguous(), **oracle_kwargs(sub))
        for key, r in ref.items():
            if r is None:
                continue
            x = got[key]
            x = x[b:b + 1, h:h + 1] if key == "dstate" else x[b:b + 1, :, h:h + 1]
            e = rel_err(x.cpu().numpy(), r)
            say(f"    b={b} h={h} {key}: rel err {e:.3e}")
            assert e <= TOL[cfg["io"]], (b, h, key, e)
    del d, got
    torch.cuda.empty_cache()
