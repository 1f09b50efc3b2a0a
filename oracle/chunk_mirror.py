"""The chunkwise WY form with absorbed decay, written literally in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: [GDN2] key design 2 ("chunk-parallel WY algorithm that absorbs the
cumulative decay").  Per chunk of C tokens, with S_[n] the state entering it:

  G_r   = sum_{i<=r} g_i (chunk-local, inclusive), gamma_r = exp(G_r)
  k_bar = k / gamma,  e_bar = gamma * e       (normalized state S_r = Diag(gamma_r) S^_r)
  T     = tril(E_bar K_bar^T, -1),  A = (I + T)^{-1}
  Y     = A E_bar,  U = A Z
  S_[n+1] = Diag(gamma_C) S_[n] + K_tail^T (U - Y S_[n])
  O_[n]   = Q_gamma S_[n] + A_qk (U - Y S_[n])

The page does not spell out K_tail, Q_gamma and A_qk.  Substituting
S_r = Diag(gamma_r) S^_r into the post-update readout o_r = S_r^T q_r gives
Q_gamma = gamma * Q, A_qk = tril(Q_gamma K_bar^T, 0) (diagonal included
because the read follows the write), and S_C = Diag(gamma_C) S^_C gives
K_tail[j] = (gamma_C / gamma_j) * k_j.  A tail chunk shorter than C is
padded with q = k = e = z = 0 and g = 0, which is the identity update.

This mirror forms gamma^{-1} literally, as the page does, so it is only used
with mild decay (|G| well inside the float64 range); it is pinned against
``oracle.recurrence`` and is used to print intermediates when debugging.
"""

from __future__ import annotations

import numpy as np

from .recurrence import _f64


def chunk_forward_one(q, k, e, z, g, S0, C=64, return_intermediates=False):
    """One (batch, head) sequence.  q, k, e [T, dk]; z [T, dv];
    g [T, dk] (log decay per key channel; broadcast a scalar decay before
    calling); S0 [dk, dv].  Returns (o [T, dv], S_final)."""
    q, k, e, z, g, S = (_f64(x) for x in (q, k, e, z, g, S0))
    S = S.copy()
    T, dk = k.shape
    dv = z.shape[1]
    n_chunks = -(-T // C)
    pad = n_chunks * C - T

    def padrows(x):
        return np.concatenate([x, np.zeros((pad,) + x.shape[1:])], axis=0) if pad else x

    q, k, e, z, g = (padrows(x) for x in (q, k, e, z, g))
    o = np.zeros((n_chunks * C, dv))
    inter = []
    for n in range(n_chunks):
        sl = slice(n * C, (n + 1) * C)
        Q, K, E, Z = q[sl], k[sl], e[sl], z[sl]
        G = np.cumsum(g[sl], axis=0)
        gam = np.exp(G)
        K_bar = K / gam
        E_bar = gam * E
        Tm = np.tril(E_bar @ K_bar.T, -1)
        A = np.linalg.inv(np.eye(C) + Tm)
        Y = A @ E_bar
        U = A @ Z
        Q_gam = gam * Q
        A_qk = np.tril(Q_gam @ K_bar.T, 0)
        K_tail = (gam[-1][None, :] / gam) * K
        W = U - Y @ S
        o[sl] = Q_gam @ S + A_qk @ W
        if return_intermediates:
            inter.append(dict(G=G, T=Tm, A=A, Y=Y, U=U, W=W, A_qk=A_qk, S_in=S.copy()))
        S = np.diag(gam[-1]) @ S + K_tail.T @ W
    o = o[:T]
    if return_intermediates:
        return o, S, inter
    return o, S


def chunk_backward_one(q, k, e, z, g, S0, do, dS_final, C=64):
    """Backward of ``chunk_forward_one`` in the chunk form's own terms
    ([GDN2] key design 3): per chunk, from the last one, with dS the gradient
    of the state leaving the chunk,

      dW   = A_qk^T dO + K_tail dS              (W = U - Y S)
      dU   = dW,  dY = -dW S^T
      dA   = dU Z^T + dY E_bar^T                (the gate-weighted dA products)
      dT   = -tril(A^T dA A^T, -1)              (adjoint of the triangular inverse)
      dE_bar = A^T dY + dT K_bar,  dZ = A^T dU,  dK_bar = dT^T E_bar + dA_qk^T Q_gamma
      dQ_gamma = dO S^T + dA_qk K_bar,  dA_qk = tril(dO W^T, 0)
      dS_in = Q_gamma^T dO + Diag(gamma_C) dS - Y^T dW

    and the decay factors gamma = exp(cumsum(g)) taken back to g by the chain
    rule (gamma^{-1} formed literally, so mild decay only, like the forward
    mirror).  Returns (dq, dk, de, dz, dg, dS0), float64, shaped like the
    inputs (de, dz: gradients of the erase directions and written values)."""
    q, k, e, z, g, S0, do, dSf = (_f64(x) for x in (q, k, e, z, g, S0, do, dS_final))
    T, dk = k.shape
    dv = z.shape[1]
    n_chunks = -(-T // C)
    pad = n_chunks * C - T

    def padrows(x):
        return np.concatenate([x, np.zeros((pad,) + x.shape[1:])], axis=0) if pad else x

    q, k, e, z, g, do = (padrows(x) for x in (q, k, e, z, g, do))
    # forward, keeping each chunk's entering state
    S_in = []
    S = S0.copy()
    for n in range(n_chunks):
        sl = slice(n * C, (n + 1) * C)
        S_in.append(S.copy())
        _, S = chunk_forward_one(q[sl], k[sl], e[sl], z[sl], g[sl], S, C=C)
    dq, dk_, de, dz, dg = (np.zeros_like(x) for x in (q, k, e, z, g))
    dS = dSf.copy()
    for n in range(n_chunks - 1, -1, -1):
        sl = slice(n * C, (n + 1) * C)
        Q, K, E, Z, dO, S = q[sl], k[sl], e[sl], z[sl], do[sl], S_in[n]
        G = np.cumsum(g[sl], axis=0)
        gam = np.exp(G)
        gC = gam[-1]
        K_bar, E_bar, Q_gam = K / gam, gam * E, gam * Q
        Tm = np.tril(E_bar @ K_bar.T, -1)
        A = np.linalg.inv(np.eye(C) + Tm)
        Y, U = A @ E_bar, A @ Z
        A_qk = np.tril(Q_gam @ K_bar.T, 0)
        K_tail = (gC[None, :] / gam) * K
        W = U - Y @ S
        # the chunk's outputs and the leaving state
        dW = A_qk.T @ dO + K_tail @ dS
        dA_qk = np.tril(dO @ W.T, 0)
        dQ_gam = dO @ S.T + dA_qk @ K_bar
        dK_tail = W @ dS.T
        dgC = np.einsum("cv,cv->c", S, dS) * gC
        dS_prev = Q_gam.T @ dO + gC[:, None] * dS - Y.T @ dW
        dU, dY = dW, -dW @ S.T
        dA = dU @ Z.T + dY @ E_bar.T
        dT = -np.tril(A.T @ dA @ A.T, -1)
        dE_bar = A.T @ dY + dT @ K_bar
        dZ = A.T @ dU
        dK_bar = dT.T @ E_bar + dA_qk.T @ Q_gam
        # back to the raw rows and the cumulative log-decay G
        dE = gam * dE_bar
        dQ = gam * dQ_gam
        dK = dK_bar / gam + dK_tail * gC[None, :] / gam
        dG = dE_bar * E_bar + dQ_gam * Q_gam - dK_bar * K_bar - dK_tail * K_tail
        dG[-1] += dgC + np.einsum("jc,jc->c", dK_tail, K_tail)
        dq[sl], dk_[sl], de[sl], dz[sl] = dQ, dK, dE, dZ
        dg[sl] = np.cumsum(dG[::-1], axis=0)[::-1]   # G = cumsum(g)
        dS = dS_prev
    return dq[:T], dk_[:T], de[:T], dz[:T], dg[:T], dS
