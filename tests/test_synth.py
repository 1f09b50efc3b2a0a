"""The seeded generator: deterministic, the right shapes, dtypes and value ranges."""

import torch

from synth import config, make_inputs


def _small(name, **kw):
    cfg = config(name, B=1, T=70, H=2, **kw)
    return make_inputs(cfg)


def test_deterministic_and_seeded():
    a = _small("gdn2_bf16_b1h32t65536d128")
    b = _small("gdn2_bf16_b1h32t65536d128")
    c = _small("gdn2_bf16_b1h32t65536d128", seed=99)
    assert torch.equal(a["k"], b["k"]) and torch.equal(a["g"], b["g"])
    assert not torch.equal(a["k"], c["k"])


def test_shapes_dtypes_ranges():
    x = _small("gdn_bf16_b8h16t4096d128")
    assert x["q"].dtype == torch.bfloat16 and x["q"].shape == (1, 70, 2, 128)
    assert x["g"].shape == (1, 70, 2) and x["g"].dtype == torch.float32 and (x["g"] <= 0).all()
    assert x["beta"].shape == (1, 70, 2) and ((x["beta"] > 0) & (x["beta"] < 1)).all()
    assert x["state"].shape == (1, 2, 128, 128)
    # q is L2-normalised and scaled by dk^-1/2, k is unit norm (up to bf16 rounding)
    qn = x["q"].float().norm(dim=-1)
    kn = x["k"].float().norm(dim=-1)
    assert ((qn - 128 ** -0.5).abs() < 1e-3).all() and ((kn - 1).abs() < 1e-2).all()
    y = _small("gdn2_bf16_b1h32t65536d128")
    assert y["b"].shape == (1, 70, 2, 128) and y["w"].shape == (1, 70, 2, 128)
    assert y["g"].shape == (1, 70, 2, 128) and y["beta"] is None
    z = _small("qdelta_bf16_b8h8t4096d128")
    assert z["lam"].shape == (2,) and z["qmix"] and ((z["lam"] >= 0) & (z["lam"] <= 1)).all()
    f = make_inputs(config("gdn_f32_b1h2t256d64"))
    assert f["q"].dtype == torch.float32 and f["state"] is None


def test_stress_knobs():
    x = _small("gdn2_bf16_b1h32t65536d128", b_scale=2.0, g_const=-20.0)
    assert (x["g"] == -20.0).all() and x["b"].max() > 1.0 and x["b"].max() <= 2.0
    y = _small("qdelta_bf16_b8h8t4096d128", lam_const=1.0, decay="none")
    assert y["g"] is None and (y["lam"] == 1.0).all()
