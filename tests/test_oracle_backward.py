"""Pins for the oracle's backward (``oracle.backward``) and output epilogue
(``oracle.epilogue``), CPU only.

The backward is pinned by central finite differences of the forward oracle
(itself pinned in ``test_oracle_pins.py``) for every input of every variant,
and the chunk form's backward of [GDN2] key design 3 (the gate-weighted dA
products and dT = -tril(A^T dA A^T, -1)) is checked against it.  The
epilogue ([CH11] §11.3: RMSNorm, then the SiLU output gate) is pinned by
torch's own rms_norm and silu in float64 and by closed forms.
"""

import inspect
import types

import numpy as np
import pytest
import torch

import oracle.backward as bwd
from oracle import gdr_recurrence
from oracle.backward import gdr_recurrence_vjp
from oracle.chunk_mirror import chunk_backward_one
from oracle.epilogue import output_norm_gate


def _unit(rng, *shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _case(variant, seed, B=2, T=9, H=2, dk=4, dv=3):
    """Inputs of one variant (kwargs of gdr_recurrence) at a tiny shape."""
    rng = np.random.default_rng(seed)
    kw = dict(q=_unit(rng, B, T, H, dk), k=_unit(rng, B, T, H, dk), v=rng.standard_normal((B, T, H, dv)),
              state=rng.standard_normal((B, H, dk, dv)) * 0.5)
    if variant in ("gdn", "qdelta", "qdelta_t", "value_beta"):
        kw.update(decay="scalar", g=-rng.uniform(0.0, 0.6, (B, T, H)))
    elif variant in ("kda", "gdn2", "value_beta_ch"):
        kw.update(decay="channel", g=-rng.uniform(0.0, 0.6, (B, T, H, dk)))
    if variant in ("value_beta", "value_beta_ch"):
        kw.update(erase="value", write="value", beta=rng.uniform(0.1, 0.9, (B, T, H, dv)))
    elif variant == "gdn2":
        kw.update(erase="channel", write="channel", b=rng.uniform(0, 2, (B, T, H, dk)),
                  w=rng.uniform(0, 1, (B, T, H, dv)))
    else:
        kw.update(beta=rng.uniform(0.1, 0.9, (B, T, H)))
    if variant == "qdelta":
        kw.update(qmix=True, lam=rng.uniform(0, 1, H))
    if variant == "qdelta_t":
        kw.update(qmix=True, lam=rng.uniform(0, 1, (B, T, H)))
    do = rng.standard_normal((B, T, H, dv))
    dS = rng.standard_normal((B, H, dk, dv))
    return kw, do, dS, rng


def _loss(kw, do, dS):
    a = dict(kw)
    o, S = gdr_recurrence(a.pop("q"), a.pop("k"), a.pop("v"), **a)
    return float((o * do).sum() + (S * dS).sum())


GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "b": "db", "w": "dw", "lam": "dlam",
           "state": "dstate"}
VARIANTS = ["deltanet", "gdn", "kda", "qdelta", "qdelta_t", "gdn2", "value_beta", "value_beta_ch"]


def _fd_check(vjp, variant, seed=0, n_idx=4, h=1e-6):
    kw, do, dS, rng = _case(variant, seed)
    grads = vjp(kw["q"], kw["k"], kw["v"], do, dstate=dS, **{x: kw[x] for x in kw if x not in "qkv"})
    worst = 0.0
    for name, gname in GRAD_OF.items():
        if name not in kw or kw[name] is None or not isinstance(kw[name], np.ndarray):
            continue
        arr = kw[name]
        scale = max(np.abs(grads[gname]).max(), 1e-3)
        for _ in range(n_idx):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            plus, minus = dict(kw), dict(kw)
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            plus[name], minus[name] = ap, am
            fd = (_loss(plus, do, dS) - _loss(minus, do, dS)) / (2 * h)
            worst = max(worst, abs(fd - grads[gname][idx]) / scale)
    return worst


@pytest.mark.parametrize("variant", VARIANTS)
def test_vjp_matches_finite_differences(variant):
    assert _fd_check(gdr_recurrence_vjp, variant) < 1e-7


def test_vjp_is_linear_in_the_cotangents():
    kw, do, dS, rng = _case("gdn2", 3)
    do2, dS2 = rng.standard_normal(do.shape), rng.standard_normal(dS.shape)
    rest = {x: kw[x] for x in kw if x not in "qkv"}
    g1 = gdr_recurrence_vjp(kw["q"], kw["k"], kw["v"], do, dstate=dS, **rest)
    g2 = gdr_recurrence_vjp(kw["q"], kw["k"], kw["v"], do2, dstate=dS2, **rest)
    g3 = gdr_recurrence_vjp(kw["q"], kw["k"], kw["v"], do + 2 * do2, dstate=dS + 2 * dS2, **rest)
    for key in ("dq", "dk", "dv", "dg", "db", "dw", "dstate"):
        np.testing.assert_allclose(g3[key], g1[key] + 2 * g2[key], rtol=1e-12, atol=1e-12)


def test_vjp_without_state_and_cotangent():
    kw, do, _, _ = _case("kda", 4)
    kw["state"] = None
    rest = {x: kw[x] for x in kw if x not in "qkv"}
    g = gdr_recurrence_vjp(kw["q"], kw["k"], kw["v"], do, **rest)
    assert g["dstate"].shape == (2, 2, 4, 3)
    kw2 = dict(kw)
    kw2["state"] = np.zeros((2, 2, 4, 3))
    rest2 = {x: kw2[x] for x in kw2 if x not in "qkv"}
    g2 = gdr_recurrence_vjp(kw2["q"], kw2["k"], kw2["v"], do, dstate=np.zeros((2, 2, 4, 3)), **rest2)
    for key in ("dq", "dk", "dv", "dg", "dbeta", "dstate"):
        np.testing.assert_array_equal(g[key], g2[key])


# planted mistakes in a private copy of oracle/backward.py: the finite
# differences must see each of them
BWD_MUTANTS = {
    "prediction_term_dropped": ("dSb = dS + e[:, :, None] * dr[:, None, :]", "dSb = dS"),
    "sign_of_dr": ("dz, dr, dm = dd, -m * dd, -r * dd", "dz, dr, dm = dd, m * dd, -r * dd"),
    "decay_grad_on_wrong_state": ("dgc = np.einsum(\"ncv,ncv->nc\", dSb, Sb)",
                                  "dgc = np.einsum(\"ncv,ncv->nc\", dSb, Sin[t])"),
    "readout_grad_transposed": ("dq[sl, t] += np.einsum(\"ncv,nv->nc\", St, dof[sl, t])",
                                "dq[sl, t] += np.einsum(\"ncv,nv->nc\", Sb, dof[sl, t])"),
    "lambda_grad_without_beta": ("dlamf[sl, t] += bef[sl, t] * np.einsum(", "dlamf[sl, t] += 1.0 * np.einsum("),
    "value_beta_dm_dropped": ("dbeta[sl, t] += dz * vf[sl, t] + dm", "dbeta[sl, t] += dz * vf[sl, t]"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_finite_differences_catch_backward_mutants(name):
    old, new = BWD_MUTANTS[name]
    src = inspect.getsource(bwd)
    assert old in src, name
    mod = types.ModuleType("bwd_mutant")
    mod.__dict__["__name__"] = "oracle.bwd_mutant"
    src = src.replace("from .recurrence import", "from oracle.recurrence import").replace(old, new)
    exec(compile(src, "bwd_mutant", "exec"), mod.__dict__)
    worst = max(_fd_check(mod.gdr_recurrence_vjp, v, n_idx=3) for v in VARIANTS)
    assert worst > 1e-4, f"{name} not detected (worst {worst:.2e})"


@pytest.mark.parametrize("variant,C,T", [("gdn2", 16, 37), ("kda", 8, 30), ("gdn", 16, 16), ("deltanet", 8, 21)])
def test_chunk_form_backward_matches_token_adjoint(variant, C, T):
    """[GDN2] key design 3 in the chunk form reaches the token adjoint."""
    kw, do, dS, _ = _case(variant, 5, B=1, T=T, H=1, dk=6, dv=5)
    rest = {x: kw[x] for x in kw if x not in "qkv"}
    gr = gdr_recurrence_vjp(kw["q"], kw["k"], kw["v"], do, dstate=dS, **rest)
    q, k, v = (kw[x][0, :, 0] for x in "qkv")
    if variant == "gdn2":
        b, w = kw["b"][0, :, 0], kw["w"][0, :, 0]
        e, z = b * k, w * v
    else:
        beta = kw["beta"][0, :, 0, None]
        e, z = beta * k, beta * v
    if variant == "deltanet":
        g = np.zeros_like(k)
    elif kw["g"].ndim == 3:
        g = np.repeat(kw["g"][0, :, 0, None], k.shape[1], axis=1)
    else:
        g = kw["g"][0, :, 0]
    cq, ck, ce, cz, cg, cS = chunk_backward_one(q, k, e, z, g, kw["state"][0, 0], do[0, :, 0], dS[0, 0], C=C)
    if variant == "gdn2":
        dk = ck + b * ce
        np.testing.assert_allclose(ce * k, gr["db"][0, :, 0], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(cz * v, gr["dw"][0, :, 0], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(cz * w, gr["dv"][0, :, 0], rtol=1e-10, atol=1e-12)
    else:
        beta = kw["beta"][0, :, 0]
        dk = ck + beta[:, None] * ce
        np.testing.assert_allclose((ce * k).sum(1) + (cz * v).sum(1), gr["dbeta"][0, :, 0], rtol=1e-10,
                                   atol=1e-12)
        np.testing.assert_allclose(beta[:, None] * cz, gr["dv"][0, :, 0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(cq, gr["dq"][0, :, 0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, gr["dk"][0, :, 0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(cS, gr["dstate"][0, 0], rtol=1e-10, atol=1e-12)
    if variant != "deltanet":
        dg = cg if kw["g"].ndim == 4 else cg.sum(1)
        gref = gr["dg"][0, :, 0]
        np.testing.assert_allclose(dg, gref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# the output epilogue


def test_epilogue_matches_torch_rms_norm_and_silu():
    rng = np.random.default_rng(70)
    o = rng.standard_normal((2, 5, 3, 16))
    gate = rng.standard_normal((2, 5, 3, 16)) * 2
    wt = rng.uniform(0.5, 1.5, 16)
    y = output_norm_gate(o, gate, wt)
    to, tg, tw = (torch.from_numpy(x) for x in (o, gate, wt))
    ref = torch.nn.functional.rms_norm(to, (16,), tw, eps=1e-6) * torch.nn.functional.silu(tg)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-15)


def test_epilogue_closed_forms():
    dv = 8
    w1 = np.ones(dv)
    # a constant row c normalises to c / sqrt(c^2 + eps)
    c = 0.3
    y = output_norm_gate(np.full((1, dv), c), np.full((1, dv), 50.0), w1, eps=0.0)
    np.testing.assert_allclose(y, np.full((1, dv), 50.0), rtol=1e-14)   # silu(50) = 50 to 1e-20
    # a zero gate closes the output; silu(-x) = silu(x) - x
    rng = np.random.default_rng(71)
    o = rng.standard_normal((4, dv))
    assert np.array_equal(output_norm_gate(o, np.zeros((4, dv)), w1), np.zeros((4, dv)))
    gt = rng.standard_normal((4, dv))
    n = output_norm_gate(o, np.ones((4, dv)) * 1e9, w1, eps=0.0) / 1e9   # the normalised row alone
    np.testing.assert_allclose(output_norm_gate(o, -gt, w1, eps=0.0),
                               output_norm_gate(o, gt, w1, eps=0.0) - n * gt, rtol=1e-12, atol=1e-12)
    # with eps = 0 the row has unit root-mean-square and is scale invariant
    np.testing.assert_allclose(np.sqrt(np.mean(n * n, axis=-1)), np.ones(4), rtol=1e-14)
    np.testing.assert_allclose(output_norm_gate(7.5 * o, gt, w1, eps=0.0), output_norm_gate(o, gt, w1, eps=0.0),
                               rtol=1e-13)
