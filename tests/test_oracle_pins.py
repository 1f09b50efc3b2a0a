"""Pins for the float64 oracle: each test checks the oracle against a fact the
pages or plain mathematics fix, never against a retyped copy of its own
formula.  CPU only.

Sources cited by title + section (see ``oracle/__init__.py`` for the full
titles): [QD] Q-Delta page, [GDN2] Gated DeltaNet-2 page, [KDA] the
"could have come up with KDA" blog, [CH11] the Gated DeltaNet book chapter.
"""

import json
import os

import numpy as np
import pytest

from oracle import gdr_recurrence
from oracle import page_forms as pf
from oracle.chunk_mirror import chunk_forward_one

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(rng, *shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _seq(x):
    """[T, d] -> [1, T, 1, d]  (or [T] -> [1, T, 1])."""
    x = np.asarray(x, dtype=np.float64)
    return x[None, :, None, ...] if x.ndim == 2 else x[None, :, None]


def _one(T, dk, dv, seed, mild=True):
    rng = np.random.default_rng(seed)
    q = _unit(rng, T, dk)
    k = _unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.05, 0.95, T)
    alpha = rng.uniform(0.7, 1.0, T) if mild else rng.uniform(0.05, 0.5, T)
    alpha_vec = rng.uniform(0.7, 1.0, (T, dk)) if mild else rng.uniform(0.05, 0.5, (T, dk))
    b = rng.uniform(0.0, 1.0, (T, dk))
    w = rng.uniform(0.0, 1.0, (T, dv))
    S0 = rng.standard_normal((dk, dv)) * 0.3
    return dict(q=q, k=k, v=v, beta=beta, alpha=alpha, alpha_vec=alpha_vec, b=b, w=w, S0=S0)


def _run(x, variant, **extra):
    """Unified oracle on one sequence given as 2-D arrays."""
    kw = dict(state=x["S0"][None, None])
    if variant == "deltanet":
        kw.update(decay="none", beta=_seq(x["beta"]))
    elif variant == "gdn":
        kw.update(decay="scalar", g=_seq(np.log(x["alpha"])), beta=_seq(x["beta"]))
    elif variant == "kda":
        kw.update(decay="channel", g=_seq(np.log(x["alpha_vec"])), beta=_seq(x["beta"]))
    elif variant == "qdelta":
        kw.update(decay="scalar", g=_seq(np.log(x["alpha"])), beta=_seq(x["beta"]), qmix=True,
                  lam=np.array([extra["lam"]]))
    elif variant == "gdn2":
        kw.update(decay="channel", g=_seq(np.log(x["alpha_vec"])), erase="channel", write="channel",
                  b=_seq(x["b"]), w=_seq(x["w"]))
    kw.update({k: v for k, v in extra.items() if k != "lam"})
    o, S = gdr_recurrence(_seq(x["q"]), _seq(x["k"]), _seq(x["v"]), **kw)
    return o[0, :, 0], S[0, 0]


def _close(a, b, tol):
    a, b = np.asarray(a), np.asarray(b)
    err = np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)
    assert err <= tol, f"relative error {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------
# P1: the worked example of [CH11] §11.2 (golden fixture)

@pytest.mark.parametrize("dv", [2, 3])
def test_worked_example_overwrites_row_exactly(dv):
    gold = json.load(open(os.path.join(GOLDEN, "ch11_worked_example.json")))
    rng = np.random.default_rng(7)
    S0 = rng.integers(-64, 64, size=(2, dv)) / 8.0  # dyadic: every product is exact
    k = np.array(gold["k"])
    v = np.array(gold["v"] + [5.0] * (dv - 2))
    o, S = gdr_recurrence(_seq(k[None])[..., :], _seq(k[None]), _seq(v[None]), decay="scalar",
                          g=np.zeros((1, 1, 1)) + np.log(gold["alpha"]),
                          beta=np.full((1, 1, 1), gold["beta"]), state=S0[None, None])
    S = S[0, 0]
    assert np.array_equal(S[0, :2], np.array(gold["row1_after"]))
    assert np.array_equal(S[0], v)
    assert np.array_equal(S[1], S0[1])          # second row untouched
    assert np.array_equal(S.T @ k, v)           # reading back along k gives v exactly
    assert np.array_equal(o[0, 0, 0], v)        # the post-update read with q = k


def test_worked_example_random_state_within_an_ulp():
    rng = np.random.default_rng(8)
    S0 = rng.standard_normal((2, 2))
    k = np.array([1.0, 0.0])
    v = np.array([3.0, 4.0])
    _, S = gdr_recurrence(_seq(k[None]), _seq(k[None]), _seq(v[None]), decay="none",
                          beta=np.ones((1, 1, 1)), state=S0[None, None])
    S = S[0, 0]
    assert np.max(np.abs(S[0] - v)) <= 2 * np.finfo(float).eps * 4
    assert np.array_equal(S[1], S0[1])


# ---------------------------------------------------------------------------
# P2: recurrence == product expansion of affine maps ([CH11] §11.4, §11.6)

@pytest.mark.parametrize("dv", [3, 2])
def test_recurrence_equals_product_expansion(dv):
    bounds = json.load(open(os.path.join(GOLDEN, "ch11_algebra_bounds.json")))
    T, dk = bounds["tokens"], bounds["dim"]
    rng = np.random.default_rng(1949)
    k = _unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    alpha = rng.uniform(0.5, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T)
    expansion = pf.product_expansion_ch11(k, v, alpha, beta)
    worst = 0.0
    for t in range(T):
        _, S = gdr_recurrence(_seq(k[:t + 1]), _seq(k[:t + 1]), _seq(v[:t + 1]), decay="scalar",
                              g=_seq(np.log(alpha[:t + 1])), beta=_seq(beta[:t + 1]))
        worst = max(worst, np.abs(S[0, 0] - expansion[t]).max())
    assert worst <= bounds["tolerance_used_here"]


def test_expansion_detects_time_order():
    """The expansion applies later transitions on the left; reversing the
    order must give a different state (so P2 can see an ordering bug)."""
    rng = np.random.default_rng(3)
    T, d = 6, 3
    k = _unit(rng, T, d)
    v = rng.standard_normal((T, d))
    alpha = rng.uniform(0.5, 1.0, T)
    beta = rng.uniform(0.2, 1.0, T)
    fwd = pf.product_expansion_ch11(k, v, alpha, beta)[-1]
    rev = pf.product_expansion_ch11(k[::-1], v[::-1], alpha[::-1], beta[::-1])[-1]
    assert np.abs(fwd - rev).max() > 1e-3


# ---------------------------------------------------------------------------
# P3: every variant against its own page's form, and the reductions between
# them ([GDN2] key design 1; [QD] key design 3 and related work; [KDA] §2.3-§4)

DK, DV, T = 5, 3, 20


def test_gdn_matches_both_page_forms():
    x = _one(T, DK, DV, 11)
    o, S = _run(x, "gdn")
    o1, S1 = pf.gdn_ch11(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"])
    o2, S2 = pf.gdn_kda(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"].T)
    _close(o, o1, 1e-13); _close(S, S1, 1e-13)
    _close(o, o2, 1e-13); _close(S, S2.T, 1e-13)


def test_deltanet_is_gdn_at_alpha_one():
    x = _one(T, DK, DV, 12)
    o, S = _run(x, "deltanet")
    o1, S1 = pf.deltanet_kda(x["q"], x["k"], x["v"], x["beta"], x["S0"].T)
    _close(o, o1, 1e-13); _close(S, S1.T, 1e-13)
    x["alpha"] = np.ones(T)
    og, Sg = _run(x, "gdn")
    _close(og, o, 1e-14); _close(Sg, S, 1e-14)


def test_kda_matches_page_form():
    x = _one(T, DK, DV, 13)
    o, S = _run(x, "kda")
    o1, S1 = pf.kda_kda(x["q"], x["k"], x["v"], x["alpha_vec"], x["beta"], x["S0"].T)
    _close(o, o1, 1e-13); _close(S, S1.T, 1e-13)


def test_kda_with_scalar_decay_is_gdn():
    x = _one(T, DK, DV, 14)
    x["alpha_vec"] = np.repeat(x["alpha"][:, None], DK, axis=1)
    o, S = _run(x, "kda")
    o1, S1 = pf.gdn_kda(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"].T)
    _close(o, o1, 1e-13); _close(S, S1.T, 1e-13)


def test_qdelta_matches_page_forms():
    x = _one(T, DK, DV, 15)
    lam = 0.37
    o, S = _run(x, "qdelta", lam=lam)
    o1, S1 = pf.qdelta_qd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], lam, x["S0"].T)
    o2, S2 = pf.qdelta_error_form(x["q"], x["k"], x["v"], x["alpha"], x["beta"], lam, x["S0"].T)
    _close(o, o1, 1e-13); _close(S, S1.T, 1e-13)
    _close(o, o2, 1e-13); _close(S, S2.T, 1e-13)


def test_qdelta_with_zero_lambda_is_gdn():
    x = _one(T, DK, DV, 16)
    o, S = _run(x, "qdelta", lam=0.0)
    o1, S1 = pf.gdn_kda(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"].T)
    _close(o, o1, 1e-13); _close(S, S1.T, 1e-13)


def test_qdelta_lambda_changes_the_result():
    x = _one(T, DK, DV, 17)
    o0, _ = _run(x, "qdelta", lam=0.0)
    o1, _ = _run(x, "qdelta", lam=0.8)
    assert np.abs(o0 - o1).max() > 1e-3


def test_gdn2_matches_page_form():
    x = _one(T, DK, DV, 18)
    x["b"] = x["b"] * 2.0  # the extended erase range of the ablation, b in [0, 2]
    o, S = _run(x, "gdn2")
    o1, S1 = pf.gdn2_gdn2(x["q"], x["k"], x["v"], x["alpha_vec"], x["b"], x["w"], x["S0"])
    _close(o, o1, 1e-13); _close(S, S1, 1e-13)


def test_gdn2_with_scalar_gates_is_kda():
    x = _one(T, DK, DV, 19)
    x["b"] = np.repeat(x["beta"][:, None], DK, axis=1)
    x["w"] = np.repeat(x["beta"][:, None], DV, axis=1)
    o, S = _run(x, "gdn2")
    o1, S1 = pf.kda_kda(x["q"], x["k"], x["v"], x["alpha_vec"], x["beta"], x["S0"].T)
    _close(o, o1, 1e-13); _close(S, S1.T, 1e-13)


# ---------------------------------------------------------------------------
# P4: Lemma 3.1 of [QD] (one-step contraction of the mixed error)

def test_qdelta_one_step_contraction():
    rng = np.random.default_rng(20)
    dk, dv = 8, 6
    checked = 0
    for trial in range(200):
        q, k = _unit(rng, 1, dk), _unit(rng, 1, dk)
        lam = rng.uniform(0, 1)
        x = k[0] + lam * q[0]
        a = k[0] @ x
        beta = rng.uniform(0.01, 1.0)
        if not (0 < beta * a < 2):
            continue
        v = rng.standard_normal((1, dv))
        S0 = rng.standard_normal((dk, dv))
        _, S1 = gdr_recurrence(_seq(q), _seq(k), _seq(v), decay="none", beta=np.full((1, 1, 1), beta),
                               qmix=True, lam=np.array([lam]), state=S0[None, None])
        S1 = S1[0, 0]
        before = np.linalg.norm(v[0] - S0.T @ x)
        after = np.linalg.norm(v[0] - S1.T @ x)
        # at alpha = 1 the contraction holds with equality: the mixed error
        # scales by exactly |1 - beta a|
        assert abs(after - abs(1 - beta * a) * before) <= 1e-12 * max(1.0, before)
        assert after <= abs(1 - beta * a) * before * (1 + 1e-12) + 1e-12
        checked += 1
    assert checked > 100


# ---------------------------------------------------------------------------
# P5: the chunk WY form of [GDN2] key design 2 reaches the recurrence exactly

@pytest.mark.parametrize("C,Tn", [(16, 100), (64, 200), (64, 64), (16, 7)])
@pytest.mark.parametrize("variant", ["gdn", "kda", "qdelta", "gdn2", "deltanet"])
def test_chunk_mirror_equals_recurrence(variant, C, Tn):
    dk, dv = 6, 4
    x = _one(Tn, dk, dv, 21 + C + Tn)
    lam = 0.6
    o_ref, S_ref = _run(x, variant, lam=lam)
    if variant in ("gdn", "qdelta"):
        g = np.repeat(np.log(x["alpha"])[:, None], dk, axis=1)
    elif variant == "deltanet":
        g = np.zeros((Tn, dk))
    else:
        g = np.log(x["alpha_vec"])
    if variant == "gdn2":
        e, z = x["b"] * x["k"], x["w"] * x["v"]
    elif variant == "qdelta":
        e, z = x["beta"][:, None] * (x["k"] + lam * x["q"]), x["beta"][:, None] * x["v"]
    else:
        e, z = x["beta"][:, None] * x["k"], x["beta"][:, None] * x["v"]
    o, S = chunk_forward_one(x["q"], x["k"], e, z, g, x["S0"], C=C)
    _close(o, o_ref, 1e-12)
    _close(S, S_ref, 1e-12)


# ---------------------------------------------------------------------------
# P6: special cases with closed forms ([CH11] §11.6 exercises; [KDA] §1.2,
# §2.1, §2.3)

def test_alpha_zero_keeps_only_the_current_write():
    x = _one(5, DK, DV, 30)
    g = np.full((5,), -np.inf)
    _, S = gdr_recurrence(_seq(x["q"]), _seq(x["k"]), _seq(x["v"]), decay="scalar", g=_seq(g),
                          beta=_seq(x["beta"]), state=x["S0"][None, None])
    expect = x["beta"][-1] * np.outer(x["k"][-1], x["v"][-1])
    _close(S[0, 0], expect, 1e-15)


def test_beta_zero_only_decays_and_still_reads():
    x = _one(5, DK, DV, 31)
    _, S = gdr_recurrence(_seq(x["q"]), _seq(x["k"]), _seq(x["v"]), decay="scalar",
                          g=_seq(np.log(x["alpha"])), beta=_seq(np.zeros(5)), state=x["S0"][None, None])
    _close(S[0, 0], np.prod(x["alpha"]) * x["S0"], 1e-14)
    o, _ = gdr_recurrence(_seq(x["q"]), _seq(x["k"]), _seq(x["v"]), decay="scalar",
                          g=_seq(np.log(x["alpha"])), beta=_seq(np.zeros(5)), state=x["S0"][None, None])
    assert np.abs(o).max() > 1e-3  # the output is not zero: the decayed state is still read


def test_no_erase_is_decayed_linear_attention():
    Tn, dk, dv = 9, 4, 3
    x = _one(Tn, dk, dv, 32)
    g = np.log(x["alpha_vec"][:, :dk])
    o, _ = gdr_recurrence(_seq(x["q"]), _seq(x["k"]), _seq(x["v"]), decay="channel", g=_seq(g),
                          erase="channel", write="channel", b=_seq(np.zeros((Tn, dk))),
                          w=_seq(x["w"]))
    ref = pf.decayed_linear_attention_bruteforce(x["q"], x["k"], x["w"] * x["v"], g)
    _close(o[0, :, 0], ref, 1e-13)


def test_no_erase_no_decay_is_linear_attention():
    Tn, dk, dv = 9, 4, 3
    x = _one(Tn, dk, dv, 33)
    o, _ = gdr_recurrence(_seq(x["q"]), _seq(x["k"]), _seq(x["v"]), decay="none",
                          erase="channel", write="channel", b=_seq(np.zeros((Tn, dk))),
                          w=_seq(np.ones((Tn, dv))))
    ref, _ = pf.linear_attention_kda(x["q"], x["k"], x["v"])
    _close(o[0, :, 0], ref, 1e-13)


def test_directions_orthogonal_to_the_key_are_untouched():
    rng = np.random.default_rng(34)
    dk, dv = 6, 4
    k = _unit(rng, 1, dk)
    xo = rng.standard_normal(dk)
    xo -= (xo @ k[0]) * k[0]  # orthogonal to k
    S0 = rng.standard_normal((dk, dv))
    _, S1 = gdr_recurrence(_seq(k), _seq(k), _seq(rng.standard_normal((1, dv))), decay="none",
                           beta=np.full((1, 1, 1), 0.7), state=S0[None, None])
    assert np.abs(xo @ (S1[0, 0] - S0)).max() <= 1e-14


def test_readback_interpolates_old_prediction_and_value():
    rng = np.random.default_rng(35)
    dk, dv = 6, 4
    k = _unit(rng, 1, dk)
    v = rng.standard_normal((1, dv))
    S0 = rng.standard_normal((dk, dv))
    beta = 0.3
    _, S1 = gdr_recurrence(_seq(k), _seq(k), _seq(v), decay="none", beta=np.full((1, 1, 1), beta),
                           state=S0[None, None])
    _close(S1[0, 0].T @ k[0], (1 - beta) * (S0.T @ k[0]) + beta * v[0], 1e-14)


# ---------------------------------------------------------------------------
# P7: [GDN2] key design 1 -- the update is the stationary point of the
# gated fast-weight objective L(S) = ||S - S_bar||^2 - 2 <S^T k, z - S_bar^T e>

def _num_grad(f, S, h=1e-5):
    G = np.zeros_like(S)
    for idx in np.ndindex(S.shape):
        Sp, Sm = S.copy(), S.copy()
        Sp[idx] += h
        Sm[idx] -= h
        G[idx] = (f(Sp) - f(Sm)) / (2 * h)
    return G


def test_gdn2_update_is_stationary_point_of_fast_weight_objective():
    rng = np.random.default_rng(36)
    dk, dv = 5, 4
    k = _unit(rng, 1, dk)
    q = _unit(rng, 1, dk)
    v = rng.standard_normal((1, dv))
    b = rng.uniform(0, 2, (1, dk))
    w = rng.uniform(0, 1, (1, dv))
    alpha = rng.uniform(0.3, 1.0, (1, dk))
    S0 = rng.standard_normal((dk, dv))
    _, S1 = gdr_recurrence(_seq(q), _seq(k), _seq(v), decay="channel", g=_seq(np.log(alpha)),
                           erase="channel", write="channel", b=_seq(b), w=_seq(w), state=S0[None, None])
    S1 = S1[0, 0]
    S_bar = alpha[0][:, None] * S0
    e, z = b[0] * k[0], w[0] * v[0]

    def L(S):
        return np.sum((S - S_bar) ** 2) - 2 * np.dot(S.T @ k[0], z - S_bar.T @ e)

    assert np.abs(_num_grad(L, S1)).max() <= 1e-8
    assert np.abs(_num_grad(L, S1 + 0.01 * rng.standard_normal(S1.shape))).max() > 1e-3


# ---------------------------------------------------------------------------
# P8: [KDA] §2.2 / [CH11] §11.2 -- DeltaNet is one gradient step of size beta
# on 0.5 ||S^T k - v||^2

def test_deltanet_is_a_gradient_step():
    rng = np.random.default_rng(37)
    dk, dv = 5, 3
    k = _unit(rng, 1, dk)
    v = rng.standard_normal((1, dv))
    S0 = rng.standard_normal((dk, dv))
    beta = 0.45
    _, S1 = gdr_recurrence(_seq(k), _seq(k), _seq(v), decay="none", beta=np.full((1, 1, 1), beta),
                           state=S0[None, None])
    grad = _num_grad(lambda S: 0.5 * np.sum((S.T @ k[0] - v[0]) ** 2), S0)
    _close(S1[0, 0], S0 - beta * grad, 1e-9)


# ---------------------------------------------------------------------------
# P9: streaming -- one call over 2L tokens equals two calls of L with the
# final state handed over ([CH11] §11.3)

@pytest.mark.parametrize("variant", ["gdn", "kda", "qdelta", "gdn2"])
def test_streaming_state_handoff(variant):
    x = _one(24, DK, DV, 40)
    o, S = _run(x, variant, lam=0.5)
    first = {key: (val[:12] if isinstance(val, np.ndarray) and val.shape[0] == 24 else val)
             for key, val in x.items()}
    second = {key: (val[12:] if isinstance(val, np.ndarray) and val.shape[0] == 24 else val)
              for key, val in x.items()}
    o1, S1 = _run(first, variant, lam=0.5)
    second["S0"] = S1
    o2, S2 = _run(second, variant, lam=0.5)
    _close(np.concatenate([o1, o2]), o, 1e-14)
    _close(S2, S, 1e-14)


def test_head_batching_does_not_change_results():
    rng = np.random.default_rng(41)
    B, Tn, H, dk, dv = 2, 10, 3, 4, 5
    q = _unit(rng, B, Tn, H, dk)
    k = _unit(rng, B, Tn, H, dk)
    v = rng.standard_normal((B, Tn, H, dv))
    g = -rng.uniform(0, 1, (B, Tn, H, dk))
    beta = rng.uniform(0, 1, (B, Tn, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    a = gdr_recurrence(q, k, v, decay="channel", g=g, beta=beta, state=S0, head_batch=64)
    c = gdr_recurrence(q, k, v, decay="channel", g=g, beta=beta, state=S0, head_batch=2)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])
    # each (b, h) pair is an independent sequence
    o1, S1 = gdr_recurrence(q[1:2, :, 2:3], k[1:2, :, 2:3], v[1:2, :, 2:3], decay="channel",
                            g=g[1:2, :, 2:3], beta=beta[1:2, :, 2:3], state=S0[1:2, 2:3])
    assert np.array_equal(o1[0, :, 0], a[0][1, :, 2]) and np.array_equal(S1[0, 0], a[1][1, 2])


# ---------------------------------------------------------------------------
# P10: a time-varying lambda_t ([QD] key design 2 writes lambda_t in [0, 1];
# key design 3 mixes it into x_t = k_t + lambda_t q_t)

def _qdelta_t(x, lam_t):
    o, S = gdr_recurrence(_seq(x["q"]), _seq(x["k"]), _seq(x["v"]), decay="scalar",
                          g=_seq(np.log(x["alpha"])), beta=_seq(x["beta"]), qmix=True,
                          lam=_seq(lam_t), state=x["S0"][None, None])
    return o[0, :, 0], S[0, 0]


def test_time_varying_lambda_matches_page_forms():
    x = _one(T, DK, DV, 50)
    lam_t = np.random.default_rng(51).uniform(0, 1, T)
    o, S = _qdelta_t(x, lam_t)
    o1, S1 = pf.qdelta_qd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], lam_t, x["S0"].T)
    o2, S2 = pf.qdelta_error_form(x["q"], x["k"], x["v"], x["alpha"], x["beta"], lam_t, x["S0"].T)
    _close(o, o1, 1e-13); _close(S, S1.T, 1e-13)
    _close(o, o2, 1e-13); _close(S, S2.T, 1e-13)


def test_constant_lambda_t_is_the_per_head_lambda():
    x = _one(T, DK, DV, 52)
    o, S = _qdelta_t(x, np.full(T, 0.37))
    o1, S1 = _run(x, "qdelta", lam=0.37)
    assert np.array_equal(o, o1) and np.array_equal(S, S1)


def test_time_varying_lambda_contracts_at_every_step():
    """Lemma 3.1 of [QD] holds token by token with x_t = k_t + lambda_t q_t:
    at alpha = 1 the mixed error of each step scales by exactly
    |1 - beta_t k_t . x_t|."""
    rng = np.random.default_rng(53)
    Tn, dk, dv = 30, 8, 6
    q, k = _unit(rng, Tn, dk), _unit(rng, Tn, dk)
    v = rng.standard_normal((Tn, dv))
    beta = rng.uniform(0.05, 0.95, Tn)
    lam_t = rng.uniform(0, 1, Tn)
    S = rng.standard_normal((dk, dv))
    for t in range(Tn):
        _, S1 = gdr_recurrence(_seq(q[t:t + 1]), _seq(k[t:t + 1]), _seq(v[t:t + 1]), decay="none",
                               beta=_seq(beta[t:t + 1]), qmix=True, lam=_seq(lam_t[t:t + 1]),
                               state=S[None, None])
        S1 = S1[0, 0]
        xt = k[t] + lam_t[t] * q[t]
        a = k[t] @ xt
        before = np.linalg.norm(v[t] - S.T @ xt)
        after = np.linalg.norm(v[t] - S1.T @ xt)
        assert abs(after - abs(1 - beta[t] * a) * before) <= 1e-12 * max(1.0, before)
        S = S1


# ---------------------------------------------------------------------------
# P11: one beta per value channel ([CH11] §11.3: the module gates each value
# channel's prediction error with its own beta; §11.4: with a vector write
# gate the affine update is read column by column of the state)

def _value_beta(x, beta_vec, decay="scalar"):
    g = np.log(x["alpha"]) if decay == "scalar" else np.log(x["alpha_vec"])
    o, S = gdr_recurrence(_seq(x["q"]), _seq(x["k"]), _seq(x["v"]), decay=decay, g=_seq(g),
                          erase="value", write="value", beta=_seq(beta_vec), state=x["S0"][None, None])
    return o[0, :, 0], S[0, 0]


def test_value_beta_matches_page_form():
    x = _one(T, DK, DV, 60)
    bv = np.random.default_rng(61).uniform(0, 1, (T, DV))
    o, S = _value_beta(x, bv)
    o1, S1 = pf.gdn_value_beta_ch11(x["q"], x["k"], x["v"], x["alpha"], bv, x["S0"])
    _close(o, o1, 1e-13); _close(S, S1, 1e-13)


@pytest.mark.parametrize("decay", ["scalar", "channel"])
def test_value_beta_is_a_scalar_beta_rule_per_column(decay):
    x = _one(T, DK, DV, 62)
    bv = np.random.default_rng(63).uniform(0, 1, (T, DV))
    o, S = _value_beta(x, bv, decay)
    for c in range(DV):
        vc, S0c = x["v"][:, c:c + 1], x["S0"][:, c:c + 1]
        if decay == "scalar":
            oc, Sc = pf.gdn_ch11(x["q"], x["k"], vc, x["alpha"], bv[:, c], S0c)
        else:
            oc, Sc = pf.kda_kda(x["q"], x["k"], vc, x["alpha_vec"], bv[:, c], S0c.T)
            Sc = Sc.T
        _close(o[:, c:c + 1], oc, 1e-13)
        _close(S[:, c:c + 1], Sc, 1e-13)


def test_value_beta_uniform_is_gated_deltanet():
    x = _one(T, DK, DV, 64)
    o, S = _value_beta(x, np.repeat(x["beta"][:, None], DV, axis=1))
    o1, S1 = pf.gdn_ch11(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"])
    _close(o, o1, 1e-13); _close(S, S1, 1e-13)


def test_value_beta_worked_example():
    """[CH11] §11.2's example with the per-channel write strength: k = e_1,
    v = [3, 4], alpha = 1, beta = [1, 1/2].  Row 1 becomes
    [3, (4 + S[0,1]) / 2] exactly (the first channel overwritten, the second
    halfway to its target); row 2 is unchanged."""
    S0 = np.array([[0.625, -1.25], [2.5, 0.375]])
    k = np.array([[1.0, 0.0]])
    v = np.array([[3.0, 4.0]])
    _, S = gdr_recurrence(_seq(k), _seq(k), _seq(v), decay="none", erase="value", write="value",
                          beta=_seq(np.array([[1.0, 0.5]])), state=S0[None, None])
    S = S[0, 0]
    assert S[0, 0] == 3.0 and S[0, 1] == (4.0 + S0[0, 1]) / 2
    assert np.array_equal(S[1], S0[1])
