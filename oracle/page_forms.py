"""Each variant written in its own page's orientation and step order.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

These functions exist to pin ``oracle.recurrence``: a test runs the unified
recurrence and the page form on the same inputs and requires agreement to
rounding.  They deliberately do NOT reuse the unified step: each one follows
the page it cites, in that page's orientation, for a single (batch, head)
sequence given as 2-D arrays [T, d] (float64).

Orientation per page:
  [KDA], [QD]    state maps key space to value space: S in R^{dv x dk},
                 prediction S k, readout S q.
  [CH11], [GDN2] state in R^{dk x dv}: prediction S^T k, readout S^T q.
"""

from __future__ import annotations

import numpy as np


def _arr(*xs):
    return [np.asarray(x, dtype=np.float64) for x in xs]


def linear_attention_kda(q, k, v):
    """[KDA] §1.1: additive write S_t = S_{t-1} + v_t k_t^T (dv x dk) and the
    read o_t = S_t q_t."""
    q, k, v = _arr(q, k, v)
    T, dk = k.shape
    S = np.zeros((v.shape[1], dk))
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        S = S + np.outer(v[t], k[t])
        o[t] = S @ q[t]
    return o, S


def deltanet_kda(q, k, v, beta, S0=None):
    """[KDA] §2.3: S_t = S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    state dv x dk, read o_t = S_t q_t."""
    q, k, v, beta = _arr(q, k, v, beta)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    eye = np.eye(dk)
    for t in range(T):
        S = S @ (eye - beta[t] * np.outer(k[t], k[t])) + beta[t] * np.outer(v[t], k[t])
        o[t] = S @ q[t]
    return o, S


def gdn_kda(q, k, v, alpha, beta, S0=None):
    """[KDA] §3 boxed Gated DeltaNet, four named steps in order:
    forget (S~ = alpha S), predict (v^ = S~ k), correct (e = beta (v - v^)),
    write (S = S~ + e k^T); state dv x dk; read o_t = S_t q_t."""
    q, k, v, alpha, beta = _arr(q, k, v, alpha, beta)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        St = alpha[t] * S
        vhat = St @ k[t]
        err = beta[t] * (v[t] - vhat)
        S = St + np.outer(err, k[t])
        o[t] = S @ q[t]
    return o, S


def gdn_ch11(q, k, v, alpha, beta, S0=None):
    """[CH11] §11.2 in dk x dv orientation: S~ = alpha S, v^ = S~^T k,
    S = S~ + beta k (v - v^)^T, read y = S^T q."""
    q, k, v, alpha, beta = _arr(q, k, v, alpha, beta)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        St = alpha[t] * S
        vhat = St.T @ k[t]
        S = St + beta[t] * np.outer(k[t], v[t] - vhat)
        o[t] = S.T @ q[t]
    return o, S


def kda_kda(q, k, v, alpha_vec, beta, S0=None, s=1.0):
    """[KDA] §4 boxed KDA: per-key-channel forget S~ = S Diag(alpha_t)
    (key channels are the columns of the dv x dk state), then predict,
    correct and write as in Gated DeltaNet; read o_t = S_t (s q_t).  The
    caller passes s = 1 when q already carries the dk^-1/2 scale."""
    q, k, v, alpha_vec, beta = _arr(q, k, v, alpha_vec, beta)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        St = S @ np.diag(alpha_vec[t])
        vhat = St @ k[t]
        err = beta[t] * (v[t] - vhat)
        S = St + np.outer(err, k[t])
        o[t] = S @ (s * q[t])
    return o, S


def _lam_at(lam, t):
    """lambda of token t: one value per head, or lambda_t ([QD] key design 2)."""
    return lam[t] if np.ndim(lam) else lam


def qdelta_qd(q, k, v, alpha, beta, lam, S0=None):
    """[QD] key design 3 (the rule rewritten with the mixed input):
    x_t = k_t + lam q_t and S_t = alpha_t S_{t-1} (I - beta_t x_t k_t^T)
    + beta_t v_t k_t^T, state dv x dk; read o_t = S_t q_t.  ``lam`` is a
    number, or one lambda_t per token (key design 2)."""
    q, k, v, alpha, beta = _arr(q, k, v, alpha, beta)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    eye = np.eye(dk)
    for t in range(T):
        x = k[t] + _lam_at(lam, t) * q[t]
        S = alpha[t] * S @ (eye - beta[t] * np.outer(x, k[t])) + beta[t] * np.outer(v[t], k[t])
        o[t] = S @ q[t]
    return o, S


def qdelta_error_form(q, k, v, alpha, beta, lam, S0=None):
    """[QD] overall framework: after forgetting, the state yields the key
    retrieval v^ = S k and the query prediction o^ = S q; the mixed error
    v - v^ - lam o^ is written back along k with strength beta (dv x dk).
    ``lam`` is a number, or one lambda_t per token."""
    q, k, v, alpha, beta = _arr(q, k, v, alpha, beta)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        S = alpha[t] * S
        vhat = S @ k[t]
        ohat = S @ q[t]
        S = S + beta[t] * np.outer(v[t] - vhat - _lam_at(lam, t) * ohat, k[t])
        o[t] = S @ q[t]
    return o, S


def gdn_value_beta_ch11(q, k, v, alpha, beta_vec, S0=None):
    """[CH11] §11.3, the module's write gate: one beta per value channel
    scales that channel's prediction error, the forget gate stays a scalar:
    S~ = alpha S, v^ = S~^T k, S = S~ + k (beta_t * (v - v^))^T (dk x dv);
    read y = S^T q."""
    q, k, v, alpha, beta_vec = _arr(q, k, v, alpha, beta_vec)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        St = alpha[t] * S
        vhat = St.T @ k[t]
        S = St + np.outer(k[t], beta_vec[t] * (v[t] - vhat))
        o[t] = S.T @ q[t]
    return o, S


def gdn2_gdn2(q, k, v, alpha_vec, b, w, S0=None):
    """[GDN2] key design 1:
    S_t = (I - k_t (b_t * k_t)^T) D_t S_{t-1} + k_t (w_t * v_t)^T, dk x dv,
    D_t = Diag(alpha_t); read o_t = S_t^T q_t."""
    q, k, v, alpha_vec, b, w = _arr(q, k, v, alpha_vec, b, w)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    eye = np.eye(dk)
    for t in range(T):
        S = (eye - np.outer(k[t], b[t] * k[t])) @ np.diag(alpha_vec[t]) @ S \
            + np.outer(k[t], w[t] * v[t])
        o[t] = S.T @ q[t]
    return o, S


def product_expansion_ch11(k, v, alpha, beta):
    """[CH11] §11.4: with A_t = alpha_t (I - beta_t k_t k_t^T) and
    U_t = beta_t k_t v_t^T, the state from zero is
    S_t = sum_i (A_t A_{t-1} ... A_{i+1}) U_i  (later factors on the left).
    Returns the list of S_1..S_T (dk x dv)."""
    k, v, alpha, beta = _arr(k, v, alpha, beta)
    T, dk = k.shape
    eye = np.eye(dk)
    A = [alpha[t] * (eye - beta[t] * np.outer(k[t], k[t])) for t in range(T)]
    U = [beta[t] * np.outer(k[t], v[t]) for t in range(T)]
    out = []
    for t in range(T):
        St = np.zeros((dk, v.shape[1]))
        for i in range(t + 1):
            P = eye.copy()
            for j in range(t, i, -1):  # A_t ... A_{i+1}, applied right to left in time
                P = P @ A[j]
            St += P @ U[i]
        out.append(St)
    return out


def decayed_linear_attention_bruteforce(q, k, z, g_vec):
    """Closed form of the rule with no erase (e = 0): each past write z_i k_i^T
    decays channel-wise until it is read, so
    o_t = sum_{i<=t} ((q_t * exp(G_t - G_i)) . k_i) z_i with G the inclusive
    cumulative log-decay ([CH11] §11.6 exercise 3: without the prediction the
    rule becomes a forgetting outer-product accumulator)."""
    q, k, z, g_vec = _arr(q, k, z, g_vec)
    T = k.shape[0]
    G = np.cumsum(g_vec, axis=0)
    o = np.zeros((T, z.shape[1]))
    for t in range(T):
        for i in range(t + 1):
            o[t] += np.dot(q[t] * np.exp(G[t] - G[i]), k[i]) * z[i]
    return o
