"""The oracle proper: the generalized gated delta rule as a plain float64
token loop.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Orientation.  The state of one (batch, head) pair is ``S`` in R^{dk x dv}:
rows are key channels, columns value channels.  A key ``k`` predicts the
value ``S^T k`` and a query reads ``S^T q``.  This is the orientation of
[GDN2] key design 1 and of [CH11] §11.1 ("a key maps to a row of readout
directions"); [QD] and [KDA] write the transpose (state maps key space to
value space), which ``page_forms`` keeps for the pins.

One step, shared by every variant the pages describe:

    forget   S_bar = D_t S_{t-1},  D_t = Diag(exp(g_t)), g_t = log(alpha_t)
    predict  r_t   = S_bar^T e_t             (read along the erase direction)
    write    S_t   = S_bar + k_t (z_t - r_t)^T
    read     o_t   = S_t^T q_t               (after the write)

Forget comes before predict ([KDA] §3 stresses that the order matters;
[CH11] §11.3 makes the same point about the decay line preceding the memory
read).  The output reads the post-update state ([CH11] §11.2 defines the
readout from S_t; the KDA box in [KDA] §4 reads S_t as well).

Variant table (e = erase/read direction, z = written value):

    DeltaNet   D = I             e = beta k            z = beta v   [KDA] §2.3
    GDN        D = alpha I       e = beta k            z = beta v   [KDA] §3, [CH11] §11.2
    KDA        D = Diag(alpha)   e = beta k            z = beta v   [KDA] §4
    Q-Delta    D = alpha I       e = beta (k + lam q)  z = beta v   [QD] key design 3
    GDN-2      D = Diag(alpha)   e = b * k             z = w * v    [GDN2] key design 1

Q-Delta: [QD] key design 3 rewrites its rule as
``S_t = alpha_t S_{t-1} (I - beta_t x_t k_t^T) + beta_t v_t k_t^T`` with the
mixed input ``x_t = k_t + lambda_t q_t`` (value-by-key orientation).
Transposed into key-by-value orientation this is the unified step with
``e = beta x`` and ``z = beta v``.  ``lam`` is one coefficient per head
([QD] key design 2 calls it a learnable per-head feedback coefficient).

GDN-2: [GDN2] key design 1 gives
``S_t = (I - k_t (b_t * k_t)^T) D_t S_{t-1} + k_t (w_t * v_t)^T``, i.e. the
unified step with ``e = b * k`` and ``z = w * v``.  The erase gate is not
clamped (the same page's ablation also trains b in [0, 2]).

Two variants of the pages go beyond that table:

* time-varying lambda: [QD] key design 2 writes the feedback coefficient as
  ``lambda_t in [0, 1]``; ``lam`` of shape [B, T, H] gives one per token
  (shape [H]: one per head, the reading the workloads use).
* one beta per value channel: [CH11] §11.3 notes that the module it follows
  gates the prediction error of each value channel with its own beta (the
  forget gate stays one scalar per head), ``S_t = S_bar + k_t (beta_t *
  (v_t - S_bar^T k_t))^T`` with ``beta_t in R^{dv}``; selected by
  ``erase = write = "value"`` with ``beta`` of shape [B, T, H, dv].  It is
  not an (e, z) pair of the table: the erase strength differs per column.
"""

from __future__ import annotations

import numpy as np

DECAYS = ("none", "scalar", "channel")
GATES = ("beta", "channel", "value")

# name -> (decay, erase, write, qmix)
VARIANTS = {
    "deltanet": ("none", "beta", "beta", False),
    "gdn": ("scalar", "beta", "beta", False),
    "kda": ("channel", "beta", "beta", False),
    "qdelta": ("scalar", "beta", "beta", True),
    "gdn2": ("channel", "channel", "channel", False),
}


def variant_kinds(name: str) -> dict:
    """Keyword arguments of ``gdr_recurrence`` that select a named variant."""
    decay, erase, write, qmix = VARIANTS[name]
    return dict(decay=decay, erase=erase, write=write, qmix=qmix)


def _f64(x):
    """Exact upcast of a numpy array or torch tensor (bf16/fp32) to float64."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor; bf16 -> float64 is exact
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _heads_first(x):
    """[B, T, H, ...] -> [B*H, T, ...]."""
    B, T, H = x.shape[:3]
    rest = x.shape[3:]
    return np.ascontiguousarray(np.moveaxis(x, 2, 1)).reshape((B * H, T) + rest)


def gdr_recurrence(q, k, v, *, decay="none", g=None, erase="beta", write="beta",
                   beta=None, b=None, w=None, qmix=False, lam=None, state=None,
                   head_batch=64):
    """Run the unified recurrence over a whole sequence.

    Shapes (all per-token tensors are [B, T, H, ...]):
      q, k      [B,T,H,dk]       v [B,T,H,dv]
      g         [B,T,H] (decay="scalar") or [B,T,H,dk] (decay="channel");
                log of the retention gate, so alpha = exp(g)
      beta      [B,T,H]          (erase and/or write == "beta", or qmix)
                [B,T,H,dv]       (erase == write == "value": one per value channel)
      b         [B,T,H,dk]       (erase == "channel")
      w         [B,T,H,dv]       (write == "channel")
      lam       [H] or [B,T,H]   (qmix; per head, or per token)
      state     [B,H,dk,dv] or None (zeros)

    Returns (o [B,T,H,dv], S_final [B,H,dk,dv]), float64 numpy arrays.
    Heads are independent ([GDN2] key design 2 has no cross-head term), so
    they are processed ``head_batch`` at a time to bound memory.
    """
    if decay not in DECAYS or erase not in GATES or write not in GATES:
        raise ValueError("bad variant kinds")
    if (erase == "value") != (write == "value"):
        raise ValueError("the per-value-channel beta gates erase and write together")
    if qmix and erase != "beta":
        raise ValueError("qmix mixes the query into a beta-gated erase direction")
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, dk = k.shape
    dv = v.shape[3]
    assert q.shape == (B, T, H, dk) and v.shape == (B, T, H, dv)

    qf, kf, vf = _heads_first(q), _heads_first(k), _heads_first(v)
    gf = _heads_first(_f64(g)) if decay != "none" else None
    bef = _heads_first(_f64(beta)) if erase != "channel" or write != "channel" else None
    bf = _heads_first(_f64(b)) if erase == "channel" else None
    wf = _heads_first(_f64(w)) if write == "channel" else None
    lamf = None
    if qmix:
        lam = _f64(lam)
        if lam.ndim == 1:  # one lambda per head, the same at every token
            lamf = np.repeat(np.repeat(lam[None, :], B, axis=0).reshape(B * H)[:, None], T, axis=1)
        else:              # lambda_t, [B, T, H]
            lamf = _heads_first(lam)
    if state is None:
        S0 = np.zeros((B * H, dk, dv))
    else:
        S0 = _f64(state).reshape(B * H, dk, dv).copy()

    o = np.zeros((B * H, T, dv))
    S_out = np.zeros((B * H, dk, dv))
    for h0 in range(0, B * H, head_batch):
        sl = slice(h0, min(B * H, h0 + head_batch))
        S = S0[sl].copy()
        for t in range(T):
            # forget
            if decay == "scalar":
                S *= np.exp(gf[sl, t])[:, None, None]
            elif decay == "channel":
                S *= np.exp(gf[sl, t])[:, :, None]
            kt = kf[sl, t]
            if erase == "value":
                # [CH11] §11.3: predict along k, gate each value channel's error
                r = np.matmul(kt[:, None, :], S)[:, 0, :]
                S += kt[:, :, None] * (bef[sl, t] * (vf[sl, t] - r))[:, None, :]
                o[sl, t] = np.matmul(qf[sl, t][:, None, :], S)[:, 0, :]
                continue
            # erase direction e and written value z
            if erase == "beta":
                x = kt + lamf[sl, t, None] * qf[sl, t] if qmix else kt
                e = bef[sl, t, None] * x
            else:
                e = bf[sl, t] * kt
            if write == "beta":
                z = bef[sl, t, None] * vf[sl, t]
            else:
                z = wf[sl, t] * vf[sl, t]
            # predict along e, then write the correction along k
            r = np.matmul(e[:, None, :], S)[:, 0, :]
            S += kt[:, :, None] * (z - r)[:, None, :]
            # read the post-update state
            o[sl, t] = np.matmul(qf[sl, t][:, None, :], S)[:, 0, :]
        S_out[sl] = S

    o = np.moveaxis(o.reshape(B, H, T, dv), 1, 2)
    return np.ascontiguousarray(o), S_out.reshape(B, H, dk, dv)


def gdr_step(q, k, v, **kw):
    """One decode step: the recurrence with T == 1 ([CH11] §11.3: a streaming
    caller keeps the final state and passes it back in on the next call)."""
    assert k.shape[1] == 1
    return gdr_recurrence(q, k, v, **kw)
