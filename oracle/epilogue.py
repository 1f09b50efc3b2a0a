"""The output epilogue of the token mixer: RMSNorm of each head's readout,
then the SiLU output gate.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[CH11] §11.3: after the readout is stacked to [B, T, H, dv], the module
applies RMSNorm and a SiLU output gate, and only then merges the heads; the
gate modulates what was read and plays no part in the state update.  [GDN2]'s
method flowchart ends with the same step ("RMSNorm and SiLU output gating").

Readings where the pages are silent: the norm runs over the dv channels of
one (batch, token, head) with a learned weight of shape [dv] shared by the
heads, eps = 1e-6, and the gate is an activation of the same shape as o:

    y = o / sqrt(mean_v(o^2) + eps) * weight * silu(gate),  silu(x) = x / (1 + exp(-x))
"""

from __future__ import annotations

import numpy as np

from .recurrence import _f64

EPS = 1e-6


def output_norm_gate(o, gate, weight, eps=EPS):
    """o, gate [..., dv]; weight [dv].  Returns y [..., dv] in float64."""
    o, gate, weight = _f64(o), _f64(gate), _f64(weight)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o / rms * weight * (gate / (1.0 + np.exp(-gate)))
