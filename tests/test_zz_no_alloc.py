"""The no-allocation chunk entry point, gdr_chunk_fwd_noalloc, called through
the C ABI and compared with gdr_chunk_fwd given a caller workspace.  Both
run the same two-pass kernels on the same inputs, the only difference being
where the records live, so the outputs must agree bitwise (which meets the
bf16 parity bar a fortiori); the smaller second call also goes against the
float64 oracle.  Two calls in a row, the second smaller, check that the
shared scratch carries nothing over from one call to the next."""

import ctypes

import pytest
import torch

import gated_delta_rule_17_amd as gdr
from gated_delta_rule_17_amd import _lib
from synth import config, make_inputs
from tests.gpu_util import TOL, assert_parity, gpu_kwargs, run_oracle, say, to_dev

pytestmark = pytest.mark.gpu

Q = "qdelta_bf16_b8h8t4096d128"
G2 = "gdn2_bf16_b1h32t65536d128"

# (larger first call, smaller second call); each takes the two-pass form
PAIRS = {
    "qdelta": (config(Q, B=2, H=8, T=1024), config(Q, B=1, H=4, T=320, decay_shift=-4.0)),
    "gdn2": (config(G2, B=1, H=8, T=2048), config(G2, B=1, H=2, T=300, decay_shift=-4.0)),
}


def _call(entry, d, ws=None):
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[3]
    o = torch.full((B, T, H, dv), float("nan"), dtype=d["q"].dtype, device=d["q"].device)
    so = torch.full((B, H, dk, dv), float("nan"), dtype=torch.float32, device=d["q"].device)
    a = gdr.build_args(d["q"], d["k"], d["v"], o=o, state_out=so, workspace=ws, **gpu_kwargs(d))
    stream = ctypes.c_void_p(torch.cuda.current_stream(d["q"].device).cuda_stream)
    _lib.call(entry, a, stream)
    return o, so


@pytest.mark.parametrize("name", sorted(PAIRS))
def test_noalloc_matches_workspace_entry_point(name):
    for i, cfg in enumerate(PAIRS[name]):
        say(f"[noalloc] {name} call {i}: B={cfg['B']} H={cfg['H']} T={cfg['T']}")
        inp = make_inputs(cfg)
        d = to_dev(inp)
        ws = gdr.new_workspace(d["q"], d["k"], d["v"], **gpu_kwargs(d))
        assert ws is not None and ws.numel() <= gdr.NOALLOC_SCRATCH_BYTES
        assert gdr.plan(d["q"], d["k"], d["v"], workspace=ws, **gpu_kwargs(d))["passes"] == 2
        o_ws, s_ws = _call("gdr_chunk_fwd", d, ws)
        o_na, s_na = _call("gdr_chunk_fwd_noalloc", d)
        torch.cuda.synchronize()
        assert torch.isfinite(o_na.float()).all() and torch.isfinite(s_na).all()
        assert torch.equal(o_na, o_ws) and torch.equal(s_na, s_ws)
        if i == 1:
            o_ref, s_ref = run_oracle(inp)
            assert_parity(f"noalloc {name}", o_na.float().cpu().numpy(), s_na.cpu().numpy(), o_ref, s_ref,
                          TOL[cfg["io"]])
