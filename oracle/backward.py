"""Gradients of the generalized gated delta rule: reverse mode through the
float64 token loop of ``oracle.recurrence``.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

For a scalar loss L with dL/do = ``do`` and dL/dS_final = ``dstate`` this
returns dL/dx for every input x of ``gdr_recurrence``.  The forward step
(same step order as the oracle, [KDA] §3 and [CH11] §11.2-§11.3) is

    S_bar = D_t S_{t-1}            D_t = Diag(exp(g_t))
    r     = S_bar^T e_t
    d     = z_t - m_t * r          m_t = 1, or beta_t in R^{dv} (per-value-channel beta)
    S_t   = S_bar + k_t d^T
    o_t   = S_t^T q_t

and its adjoint, token by token from the last one, with dS the running
gradient of the state:

    dS    += q_t do_t^T ;          dq_t += S_t do_t
    dk_t  += dS d ;                dd    = dS^T k_t
    dz_t   = dd ;  dr = -m_t * dd ; dm_t = -r * dd
    dS_bar = dS + e_t dr^T ;       de_t  = S_bar dr
    dg_t   = rowsum(dS_bar * S_bar) (summed over channels for a scalar decay)
    dS     = D_t dS_bar            (the gradient of S_{t-1})

then through the gates: e = beta (k + lambda q) gives dbeta += de . x,
dk += beta de, dq += beta lambda de, dlambda += beta de . q; e = b * k gives
db = de * k, dk += b * de; z = beta v gives dbeta += dz . v, dv = beta dz;
z = w * v gives dw = dz * v, dv = w * dz; the per-value-channel beta
(e = k, z = beta * v, m = beta) gives dbeta = dz * v + dm, dv = beta * dz.
A lambda shared by the tokens of a head sums its per-token gradients.

[GDN2] key design 3 gives the chunk form's version of the same backward
(gate weights inside the dA products, dT = -tril(A^T dA A^T, -1));
``oracle.chunk_mirror.chunk_backward_one`` writes that form literally and a
pin checks it against this token-level adjoint, which itself is pinned by
finite differences of the forward oracle.
"""

from __future__ import annotations

import numpy as np

from .recurrence import DECAYS, GATES, _f64, _heads_first


def _heads_last(x, B, H):
    """[B*H, T, ...] -> [B, T, H, ...]."""
    rest = x.shape[2:]
    return np.ascontiguousarray(np.moveaxis(x.reshape((B, H) + x.shape[1:]), 1, 2)).reshape(
        (B, x.shape[1], H) + rest)


def gdr_recurrence_vjp(q, k, v, do, *, dstate=None, decay="none", g=None, erase="beta", write="beta",
                       beta=None, b=None, w=None, qmix=False, lam=None, state=None, head_batch=16):
    """Gradients of L = <do, o> + <dstate, S_final>.

    Arguments as ``oracle.gdr_recurrence``, plus ``do`` [B,T,H,dv] and
    ``dstate`` [B,H,dk,dv] (None = 0).  Returns a dict of float64 arrays
    shaped like the inputs: dq, dk, dv, dg (None without decay), dbeta, db,
    dw, dlam (None where the input is unused) and dstate (the gradient of
    the initial state, shaped [B,H,dk,dv] whether or not one was given).
    """
    if decay not in DECAYS or erase not in GATES or write not in GATES:
        raise ValueError("bad variant kinds")
    if (erase == "value") != (write == "value"):
        raise ValueError("the per-value-channel beta gates erase and write together")
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, T, H, dk = k.shape
    dv = v.shape[3]
    BH = B * H
    qf, kf, vf, dof = _heads_first(q), _heads_first(k), _heads_first(v), _heads_first(do)
    gf = _heads_first(_f64(g)) if decay != "none" else None
    need_beta = erase != "channel" or write != "channel"
    bef = _heads_first(_f64(beta)) if need_beta else None
    bf = _heads_first(_f64(b)) if erase == "channel" else None
    wf = _heads_first(_f64(w)) if write == "channel" else None
    lam_per_head = False
    lamf = None
    if qmix:
        lam = _f64(lam)
        lam_per_head = lam.ndim == 1
        lamf = (np.repeat(np.repeat(lam[None, :], B, axis=0).reshape(BH)[:, None], T, axis=1)
                if lam_per_head else _heads_first(lam))
    S0 = np.zeros((BH, dk, dv)) if state is None else _f64(state).reshape(BH, dk, dv)
    dSf = np.zeros((BH, dk, dv)) if dstate is None else _f64(dstate).reshape(BH, dk, dv)

    dq, dkk, dvv = np.zeros_like(qf), np.zeros_like(kf), np.zeros_like(vf)
    dg = np.zeros_like(gf) if gf is not None else None
    dbeta = np.zeros_like(bef) if bef is not None else None
    db = np.zeros_like(bf) if bf is not None else None
    dw = np.zeros_like(wf) if wf is not None else None
    dlamf = np.zeros((BH, T)) if qmix else None
    dS0 = np.zeros((BH, dk, dv))

    for h0 in range(0, BH, head_batch):
        sl = slice(h0, min(BH, h0 + head_batch))
        nb = sl.stop - sl.start

        def gates(t):
            """(D [nb, dk], e, x, z, m) of token t for the heads in ``sl``."""
            if decay == "scalar":
                D = np.repeat(np.exp(gf[sl, t])[:, None], dk, axis=1)
            elif decay == "channel":
                D = np.exp(gf[sl, t])
            else:
                D = np.ones((nb, dk))
            kt = kf[sl, t]
            x = None
            if erase == "value":
                e, m, z = kt, bef[sl, t], bef[sl, t] * vf[sl, t]
            else:
                if erase == "beta":
                    x = kt + lamf[sl, t, None] * qf[sl, t] if qmix else kt
                    e = bef[sl, t, None] * x
                else:
                    e = bf[sl, t] * kt
                m = np.ones((nb, dv))
                z = bef[sl, t, None] * vf[sl, t] if write == "beta" else wf[sl, t] * vf[sl, t]
            return D, e, x, z, m

        # forward, keeping the state that enters every token
        Sin = np.zeros((T + 1, nb, dk, dv))
        S = S0[sl].copy()
        for t in range(T):
            Sin[t] = S
            D, e, _, z, m = gates(t)
            Sb = D[:, :, None] * S
            r = np.einsum("nc,ncv->nv", e, Sb)
            S = Sb + kf[sl, t][:, :, None] * (z - m * r)[:, None, :]
        Sin[T] = S

        # reverse
        dS = dSf[sl].copy()
        for t in range(T - 1, -1, -1):
            D, e, x, z, m = gates(t)
            kt, qt = kf[sl, t], qf[sl, t]
            Sb = D[:, :, None] * Sin[t]
            r = np.einsum("nc,ncv->nv", e, Sb)
            d = z - m * r
            St = Sb + kt[:, :, None] * d[:, None, :]
            # o_t = S_t^T q_t
            dS += qt[:, :, None] * dof[sl, t][:, None, :]
            dq[sl, t] += np.einsum("ncv,nv->nc", St, dof[sl, t])
            # S_t = S_bar + k d^T
            dkt = np.einsum("ncv,nv->nc", dS, d)
            dd = np.einsum("ncv,nc->nv", dS, kt)
            dz, dr, dm = dd, -m * dd, -r * dd
            # r = S_bar^T e
            dSb = dS + e[:, :, None] * dr[:, None, :]
            de = np.einsum("ncv,nv->nc", Sb, dr)
            # S_bar = D S_{t-1}
            dgc = np.einsum("ncv,ncv->nc", dSb, Sb)
            if decay == "scalar":
                dg[sl, t] = dgc.sum(axis=1)
            elif decay == "channel":
                dg[sl, t] = dgc
            dS = D[:, :, None] * dSb
            # erase side
            if erase == "value":
                dkt = dkt + de
                dbeta[sl, t] += dz * vf[sl, t] + dm
                dvv[sl, t] += bef[sl, t] * dz
            else:
                if erase == "beta":
                    dbeta[sl, t] += np.einsum("nc,nc->n", de, x)
                    bt = bef[sl, t, None]
                    dkt = dkt + bt * de
                    if qmix:
                        dq[sl, t] += bt * lamf[sl, t, None] * de
                        dlamf[sl, t] += bef[sl, t] * np.einsum("nc,nc->n", de, qt)
                else:
                    db[sl, t] += de * kt
                    dkt = dkt + bf[sl, t] * de
                # write side
                if write == "beta":
                    dbeta[sl, t] += np.einsum("nv,nv->n", dz, vf[sl, t])
                    dvv[sl, t] += bef[sl, t, None] * dz
                else:
                    dw[sl, t] += dz * vf[sl, t]
                    dvv[sl, t] += wf[sl, t] * dz
            dkk[sl, t] += dkt
        dS0[sl] = dS

    out = dict(dq=_heads_last(dq, B, H), dk=_heads_last(dkk, B, H), dv=_heads_last(dvv, B, H),
               dg=_heads_last(dg, B, H) if dg is not None else None,
               dbeta=_heads_last(dbeta, B, H) if dbeta is not None else None,
               db=_heads_last(db, B, H) if db is not None else None,
               dw=_heads_last(dw, B, H) if dw is not None else None,
               dlam=None, dstate=dS0.reshape(B, H, dk, dv))
    if qmix:
        dl = _heads_last(dlamf, B, H)  # [B, T, H]
        out["dlam"] = dl.sum(axis=(0, 1)) if lam_per_head else dl
    return out
