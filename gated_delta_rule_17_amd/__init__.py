"""Python binding of libgdr: the chunkwise gated delta rule forward and its
decode step on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/gdr.h``.  PyTorch provides device
memory and the current stream.  There is no CPU fallback: if the shared
library is missing, importing the functions raises.

    o, state = chunk_fwd(q, k, v, g=g, beta=beta, state=S0)          # GDN
    o, state = chunk_fwd(q, k, v, g=g_channel, beta=beta)            # KDA
    o, state = chunk_fwd(q, k, v, g=g, beta=beta, lam=lam)           # Q-Delta
    o, state = chunk_fwd(q, k, v, g=g_channel, b=b, w=w)             # Gated DeltaNet-2
    o, state = chunk_fwd(q, k, v, g=g, beta=beta, lam=lam_t)         # Q-Delta, lambda_t [B,T,H]
    o, state = chunk_fwd(q, k, v, g=g, beta=beta_v)                  # beta per value channel [B,T,H,dv]
    o, state = recurrent_step(q1, k1, v1, ..., state=state)          # one token
    o, state = recurrent_fwd(q, k, v, ..., state=state)              # token loop, short T
    y, state = chunk_fwd(..., gate=gate, norm_weight=wt)             # + RMSNorm, SiLU gate
    y = output_norm_gate(o, gate, wt)                                # the epilogue alone
    grads = chunk_bwd(q, k, v, do, g=g, beta=beta, state=S0, dstate=dS)  # backward

Shapes: q, k [B,T,H,dk]; v [B,T,H,dv]; g [B,T,H] (scalar decay) or
[B,T,H,dk] (per-channel decay); beta [B,T,H] (or [B,T,H,dv]: one beta per
value channel); b [B,T,H,dk]; w [B,T,H,dv]; lam [H] (or [B,T,H]: lambda_t);
state [B,H,dk,dv] fp32.  Returns o [B,T,H,dv] in q's dtype and the final
state [B,H,dk,dv] fp32.
"""

from __future__ import annotations

import ctypes
import os

import torch

from . import _lib
from ._lib import GdrArgs, GdrBwdArgs, GdrNormArgs, GdrPlanInfo, GdrError  # noqa: F401

DTYPES = {torch.float32: 0, torch.bfloat16: 1}
# bytes of the library's own scratch used by chunk_fwd_noalloc (per device)
NOALLOC_SCRATCH_BYTES = 64 << 20
DECAY = {"none": 0, "scalar": 1, "channel": 2}
GATE = {"beta": 0, "channel": 1, "value": 2}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _fptr(t):
    return ctypes.cast(ctypes.c_void_p(t.data_ptr()), ctypes.POINTER(ctypes.c_float)) if t is not None \
        else ctypes.POINTER(ctypes.c_float)()


def _check(t, name, dtype=None, ndim=None, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def build_args(q, k, v, *, g=None, beta=None, b=None, w=None, lam=None, state=None,
               o=None, state_out=None, decay=None, erase=None, write=None, qmix=None,
               dv_split=0, T=None, workspace=None, gate=None, norm_weight=None, norm_eps=0.0):
    """Fill a ``gdr_args`` struct from tensors (no device work).  Kinds are
    inferred from which gates are given unless passed explicitly.
    ``workspace``: an optional uint8 device tensor for the two-pass form.
    ``gate``, ``norm_weight``, ``norm_eps``: the optional output epilogue."""
    B, Tq, H, dk = q.shape
    dv = v.shape[3]
    vbeta = beta is not None and beta.dim() == 4
    if decay is None:
        decay = "none" if g is None else ("scalar" if g.dim() == 3 else "channel")
    if erase is None:
        erase = "value" if vbeta else ("channel" if b is not None else "beta")
    if write is None:
        write = "value" if vbeta else ("channel" if w is not None else "beta")
    if qmix is None:
        qmix = 0 if lam is None else (2 if lam.dim() == 3 else 1)
    a = GdrArgs()
    a.struct_size = ctypes.sizeof(GdrArgs)
    a.B, a.T, a.H, a.dk, a.dv = B, Tq if T is None else T, H, dk, dv
    a.chunk = 64
    a.io = DTYPES[q.dtype]
    qm = int(qmix)
    if qm == 1 and lam is not None and lam.dim() == 3:
        qm = 2
    a.decay, a.erase, a.write, a.qmix = DECAY[decay], GATE[erase], GATE[write], qm
    a.dv_split = int(dv_split)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.g, a.beta, a.b, a.w, a.lambda_ = _fptr(g), _fptr(beta), _fptr(b), _fptr(w), _fptr(lam)
    a.state_in = _fptr(state)
    a.state_out = _fptr(state_out)
    a.o = _ptr(o)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel() if workspace is not None else 0
    a.out_gate = _ptr(gate)
    a.norm_weight = _fptr(norm_weight)
    a.norm_eps = float(norm_eps)
    return a


def workspace_size(q, k, v, **kw) -> int:
    """Bytes of workspace that ``chunk_fwd`` with these tensors can use for
    its two-pass form (0 when the shape takes the single pass); host-only."""
    a = build_args(q, k, v, **kw)
    n = ctypes.c_uint64(0)
    _lib.call("gdr_workspace_size", a, ctypes.byref(n))
    return int(n.value)


def new_workspace(q, k, v, **kw):
    """A uint8 device tensor of ``workspace_size`` bytes, or None."""
    n = workspace_size(q, k, v, **kw)
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n else None


def _check_epilogue(q, v, gate, norm_weight):
    if gate is None:
        return
    _check(gate, "gate", dtype=q.dtype, ndim=4, device=q.device)
    _check(norm_weight, "norm_weight", dtype=torch.float32, ndim=1, device=q.device)
    if gate.shape != v.shape or norm_weight.shape[0] != v.shape[3]:
        raise ValueError(f"gate must be shaped like v {tuple(v.shape)} and norm_weight [dv]")


def _prepare(q, k, v, g, beta, b, w, lam, state, decay=None):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    if q.dtype not in DTYPES:
        raise TypeError(f"q must be bf16 or fp32, got {q.dtype}")
    _check(q, "q", ndim=4, device=dev)
    _check(k, "k", dtype=q.dtype, ndim=4, device=dev)
    _check(v, "v", dtype=q.dtype, ndim=4, device=dev)
    for name, t in (("g", g), ("beta", beta), ("b", b), ("w", w), ("lam", lam), ("state", state)):
        _check(t, name, dtype=torch.float32, device=dev)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != (B, T, H):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if g is not None and tuple(g.shape) not in ((B, T, H), (B, T, H, dk)):
        raise ValueError(f"g must be [B,T,H] or [B,T,H,dk], got {tuple(g.shape)}")
    if g is not None and decay is not None:
        want = {"scalar": 3, "channel": 4}.get(decay)
        if want != g.dim():
            raise ValueError(f"decay={decay!r} needs g with {want} dims, got shape {tuple(g.shape)}")
    if beta is not None and tuple(beta.shape) not in ((B, T, H), (B, T, H, dv)):
        raise ValueError(f"beta must be [B,T,H] or [B,T,H,dv], got {tuple(beta.shape)}")
    if b is not None and tuple(b.shape) != (B, T, H, dk):
        raise ValueError(f"b must be [B,T,H,dk], got {tuple(b.shape)}")
    if w is not None and tuple(w.shape) != (B, T, H, dv):
        raise ValueError(f"w must be [B,T,H,dv], got {tuple(w.shape)}")
    if lam is not None and tuple(lam.shape) not in ((H,), (B, T, H)):
        raise ValueError(f"lam must be [H] or [B,T,H], got {tuple(lam.shape)}")
    if state is not None and tuple(state.shape) != (B, H, dk, dv):
        raise ValueError(f"state must be [B,H,dk,dv], got {tuple(state.shape)}")
    return B, T, H, dk, dv


def _stream_ptr(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def chunk_fwd(q, k, v, *, g=None, beta=None, b=None, w=None, lam=None, state=None,
              decay=None, erase=None, write=None, qmix=None, dv_split=0,
              out=None, state_out=None, workspace=None, two_pass=None,
              gate=None, norm_weight=None, norm_eps=0.0):
    """Chunkwise forward (C = 64) of the generalized gated delta rule.
    Enqueued on the current stream; no synchronisation.

    ``workspace``: a uint8 device tensor of at least ``workspace_size()``
    bytes (see ``new_workspace``) selects the two-pass form where the library
    offers one; a smaller one raises.  Without one the call allocates nothing
    but its outputs (unless ``out``/``state_out`` are given too).
    ``two_pass``: None lets the workspace decide; False never uses the
    two-pass form; True requires it and, when no workspace is passed,
    allocates one for this call.
    ``gate``, ``norm_weight``: the output epilogue (RMSNorm, SiLU gate);
    the returned tensor then holds y instead of the readout."""
    B, T, H, dk, dv = _prepare(q, k, v, g, beta, b, w, lam, state, decay)
    _check_epilogue(q, v, gate, norm_weight)
    o = out if out is not None else torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    so = state_out if state_out is not None else torch.empty((B, H, dk, dv), dtype=torch.float32,
                                                             device=q.device)
    kw = dict(g=g, beta=beta, b=b, w=w, lam=lam, state=state, decay=decay, erase=erase, write=write,
              qmix=qmix, dv_split=dv_split)
    ws = None
    if two_pass is not False and (two_pass or workspace is not None):
        need = workspace_size(q, k, v, **kw)
        if two_pass and not need:
            raise ValueError("this shape has no two-pass form")
        if need:
            _check(workspace, "workspace", dtype=torch.uint8, ndim=1, device=q.device)
            if workspace is None:
                ws = torch.empty(need, dtype=torch.uint8, device=q.device)
            elif workspace.numel() < need:
                raise ValueError(f"workspace has {workspace.numel()} bytes, the two-pass form needs {need}")
            else:
                ws = workspace
    a = build_args(q, k, v, o=o, state_out=so, workspace=ws, gate=gate, norm_weight=norm_weight,
                   norm_eps=norm_eps, **kw)
    _lib.call("gdr_chunk_fwd", a, _stream_ptr(q.device))
    return o, so


def chunk_fwd_noalloc(q, k, v, *, g=None, beta=None, b=None, w=None, lam=None, state=None,
                      decay=None, erase=None, write=None, qmix=None, dv_split=0, out=None, state_out=None):
    """``gdr_chunk_fwd_noalloc``: the chunkwise forward with the two-pass
    records in the library's static scratch (NOALLOC_SCRATCH_BYTES per
    device) instead of a workspace.  With ``out`` and ``state_out`` given,
    nothing is allocated; calls that overlap on one GPU race on the scratch."""
    B, T, H, dk, dv = _prepare(q, k, v, g, beta, b, w, lam, state, decay)
    o = out if out is not None else torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    so = state_out if state_out is not None else torch.empty((B, H, dk, dv), dtype=torch.float32,
                                                             device=q.device)
    a = build_args(q, k, v, g=g, beta=beta, b=b, w=w, lam=lam, state=state, o=o, state_out=so,
                   decay=decay, erase=erase, write=write, qmix=qmix, dv_split=dv_split)
    _lib.call("gdr_chunk_fwd_noalloc", a, _stream_ptr(q.device))
    return o, so


def recurrent_step(q, k, v, *, g=None, beta=None, b=None, w=None, lam=None, state=None,
                   decay=None, erase=None, write=None, qmix=None, out=None, state_out=None,
                   gate=None, norm_weight=None, norm_eps=0.0):
    """One decode token (T == 1).  ``state_out`` may be ``state`` itself for
    an in-place update."""
    B, T, H, dk, dv = _prepare(q, k, v, g, beta, b, w, lam, state, decay)
    _check_epilogue(q, v, gate, norm_weight)
    if T != 1:
        raise ValueError("recurrent_step takes exactly one token (T == 1)")
    o = out if out is not None else torch.empty((B, 1, H, dv), dtype=q.dtype, device=q.device)
    so = state_out if state_out is not None else torch.empty((B, H, dk, dv), dtype=torch.float32,
                                                             device=q.device)
    a = build_args(q, k, v, g=g, beta=beta, b=b, w=w, lam=lam, state=state, o=o, state_out=so,
                   decay=decay, erase=erase, write=write, qmix=qmix, gate=gate, norm_weight=norm_weight,
                   norm_eps=norm_eps)
    _lib.call("gdr_recurrent_step", a, _stream_ptr(q.device))
    return o, so


def recurrent_fwd(q, k, v, *, g=None, beta=None, b=None, w=None, lam=None, state=None,
                  decay=None, erase=None, write=None, qmix=None, out=None, state_out=None,
                  gate=None, norm_weight=None, norm_eps=0.0):
    """``gdr_recurrent_fwd``: the token loop in one kernel over any T (short
    sequences), the state in registers; same arguments as ``chunk_fwd``."""
    B, T, H, dk, dv = _prepare(q, k, v, g, beta, b, w, lam, state, decay)
    _check_epilogue(q, v, gate, norm_weight)
    o = out if out is not None else torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    so = state_out if state_out is not None else torch.empty((B, H, dk, dv), dtype=torch.float32,
                                                             device=q.device)
    a = build_args(q, k, v, g=g, beta=beta, b=b, w=w, lam=lam, state=state, o=o, state_out=so,
                   decay=decay, erase=erase, write=write, qmix=qmix, gate=gate, norm_weight=norm_weight,
                   norm_eps=norm_eps)
    _lib.call("gdr_recurrent_fwd", a, _stream_ptr(q.device))
    return o, so


def build_bwd_args(fwd_args, do, *, dstate=None, grads=None, workspace=None):
    """Fill a ``gdr_bwd_args`` struct (no device work).  ``fwd_args`` is a
    ``GdrArgs`` from ``build_args`` (kept alive by the caller); ``grads`` a
    dict of fp32 output tensors (dq, dk, dv, dg, dbeta, db, dw, dlam, dstate)."""
    grads = grads or {}
    a = GdrBwdArgs()
    a.struct_size = ctypes.sizeof(GdrBwdArgs)
    a.fwd = ctypes.pointer(fwd_args)
    a.d_o = _ptr(do)
    a.d_state = _fptr(dstate)
    for name in ("dq", "dk", "dv", "dg", "dbeta", "db", "dw", "dlam", "dstate"):
        setattr(a, name, _fptr(grads.get(name)))
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel() if workspace is not None else 0
    return a


def bwd_workspace_size(q, k, v, do, **kw) -> int:
    """Bytes of workspace ``chunk_bwd`` needs with these tensors (host-only)."""
    fa = build_args(q, k, v, o=do, **kw)
    a = build_bwd_args(fa, do)
    n = ctypes.c_uint64(0)
    _lib.call("gdr_bwd_workspace_size", a, ctypes.byref(n))
    return int(n.value)


def chunk_bwd(q, k, v, do, *, g=None, beta=None, b=None, w=None, lam=None, state=None, dstate=None,
              decay=None, erase=None, write=None, qmix=None, grads=None, workspace=None):
    """``gdr_chunk_bwd``: gradients of every input of ``chunk_fwd`` for the
    cotangents ``do`` (of o, shaped like v, q's dtype) and ``dstate`` (of the
    final state, or None).  Returns a dict of fp32 tensors dq, dk, dv and,
    where the forward uses them, dg, dbeta, db, dw, dlam, and dstate (the
    gradient of ``state``).  ``grads``: preallocated outputs by name;
    ``workspace``: a uint8 device tensor of ``bwd_workspace_size()`` bytes
    (allocated for this call when not given)."""
    B, T, H, dk, dv = _prepare(q, k, v, g, beta, b, w, lam, state, decay)
    _check(do, "do", dtype=q.dtype, ndim=4, device=q.device)
    _check(dstate, "dstate", dtype=torch.float32, device=q.device)
    if do.shape != v.shape:
        raise ValueError(f"do must be shaped like v {tuple(v.shape)}")
    kw = dict(g=g, beta=beta, b=b, w=w, lam=lam, state=state, decay=decay, erase=erase, write=write, qmix=qmix)
    fa = build_args(q, k, v, o=do, **kw)
    f32 = dict(dtype=torch.float32, device=q.device)
    out = dict(grads or {})
    out.setdefault("dq", torch.empty((B, T, H, dk), **f32))
    out.setdefault("dk", torch.empty((B, T, H, dk), **f32))
    out.setdefault("dv", torch.empty((B, T, H, dv), **f32))
    out.setdefault("dstate", torch.empty((B, H, dk, dv), **f32))
    for name, src in (("dg", g), ("db", b), ("dw", w), ("dlam", lam)):
        if src is not None:
            out.setdefault(name, torch.empty(src.shape, **f32))
    if fa.erase == 0 or fa.write == 0:
        out.setdefault("dbeta", torch.empty((B, T, H), **f32))
    need = bwd_workspace_size(q, k, v, do, **kw)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    a = build_bwd_args(fa, do, dstate=dstate, grads=out, workspace=workspace)
    _lib.call("gdr_chunk_bwd", a, _stream_ptr(q.device))
    return out


def output_norm_gate(o, gate, weight, *, eps=0.0, out=None):
    """``gdr_output_norm_gate``: y = RMSNorm(o) * weight * silu(gate) over the
    last dimension of o (any leading shape); ``out`` may be ``o`` (in place)."""
    if o.device.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    _check(o, "o", device=o.device)
    _check(gate, "gate", dtype=o.dtype, device=o.device)
    _check(weight, "weight", dtype=torch.float32, ndim=1, device=o.device)
    if gate.shape != o.shape or weight.shape[0] != o.shape[-1]:
        raise ValueError("gate must be shaped like o and weight [dv]")
    y = out if out is not None else torch.empty_like(o)
    a = GdrNormArgs()
    a.struct_size = ctypes.sizeof(GdrNormArgs)
    a.dv = o.shape[-1]
    a.io = DTYPES[o.dtype]
    a.eps = float(eps)
    a.rows = o.numel() // o.shape[-1] if o.numel() else 0
    a.o, a.gate, a.y = _ptr(o), _ptr(gate), _ptr(y)
    a.weight = _fptr(weight)
    _lib.call("gdr_output_norm_gate", a, _stream_ptr(o.device))
    return y


def plan(q, k, v, op="chunk", **kw):
    """Launch plan (grid, block, value-slice width, LDS bytes, chunks) that a
    call with these tensors would use; host-only."""
    a = build_args(q, k, v, **kw)
    info = GdrPlanInfo()
    _lib.call("gdr_plan", a, {"chunk": 0, "step": 1, "recurrent": 2}[op], ctypes.byref(info))
    return dict(grid=info.grid, block=info.block, dv_slice=info.dv_slice, lds_bytes=info.lds_bytes,
                n_chunks=info.n_chunks, passes=info.passes)


def library_path() -> str:
    return _lib.path()


__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "recurrent_step", "recurrent_fwd",
           "output_norm_gate", "chunk_bwd", "bwd_workspace_size", "build_bwd_args", "plan", "build_args", "workspace_size", "new_workspace",
           "library_path", "GdrError"]
