"""C-ABI checks that run without a GPU: the library loads, exports every
function ``include/gdr.h`` declares, and rejects bad arguments in host
validation (before any HIP call; the pointers below are never dereferenced)."""

import ctypes
import os
import re
import subprocess

import pytest

from gated_delta_rule_17_amd import _lib
from gated_delta_rule_17_amd._lib import GdrArgs, GdrNormArgs, GdrPlanInfo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_UNSUP, E_HIP, E_ARGS = range(8)
CHUNK, STEP, RECUR = 0, 1, 2


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_]+)\s*\(", src)))


def test_header_functions_are_exported(lib):
    declared = _declared_functions()
    assert set(declared) >= {"gdr_chunk_fwd", "gdr_recurrent_step", "gdr_status_str",
                             "gdr_last_error", "gdr_abi_version", "gdr_validate", "gdr_plan",
                             "gdr_workspace_size"}
    for name in declared:
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.path()], capture_output=True, text=True)
    if nm.returncode == 0:
        exported = set(re.findall(r" T (gdr_\w+)", nm.stdout))
        assert set(declared) <= exported
    assert sorted(_lib.EXPORTS) == declared


def test_abi_version_and_status_strings(lib):
    assert lib.gdr_abi_version() == 3
    for code, name in _lib.STATUS.items():
        assert lib.gdr_status_str(code).decode() == name
    assert lib.gdr_status_str(99).decode() == "GDR_E_UNKNOWN"


# fake, aligned, non-overlapping addresses (validation never dereferences them)
_BASE = 0x7F0000000000
_STEP = 1 << 32


def _addr(i, off=0):
    return _BASE + i * _STEP + off


def good_args(**kw):
    a = GdrArgs()
    a.struct_size = ctypes.sizeof(GdrArgs)
    a.B, a.T, a.H, a.dk, a.dv = 2, 200, 4, 128, 128
    a.chunk, a.io, a.decay, a.erase, a.write, a.qmix, a.dv_split = 64, 1, 1, 0, 0, 0, 0
    fp = ctypes.POINTER(ctypes.c_float)
    a.q, a.k, a.v, a.o = _addr(0), _addr(1), _addr(2), _addr(3)
    a.g = ctypes.cast(ctypes.c_void_p(_addr(4)), fp)
    a.beta = ctypes.cast(ctypes.c_void_p(_addr(5)), fp)
    a.state_in = ctypes.cast(ctypes.c_void_p(_addr(6)), fp)
    a.state_out = ctypes.cast(ctypes.c_void_p(_addr(7)), fp)
    for key, val in kw.items():
        if key in ("g", "beta", "b", "w", "lambda_", "state_in", "state_out"):
            val = ctypes.cast(ctypes.c_void_p(val), fp) if val else fp()
        setattr(a, key, val)
    return a


def _validate(lib, a, op=CHUNK):
    return lib.gdr_validate(ctypes.byref(a), op)


def test_good_args_validate(lib):
    assert _validate(lib, good_args()) == OK
    assert _validate(lib, good_args(T=1), STEP) == OK


def test_null_struct(lib):
    assert lib.gdr_validate(None, CHUNK) == E_NULL
    assert lib.gdr_chunk_fwd(None, None) == E_NULL
    assert b"NULL" in lib.gdr_last_error()


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 8, E_ARGS),
    ("B", 0, E_SHAPE), ("H", 0, E_SHAPE), ("T", -1, E_SHAPE),
    ("chunk", 32, E_SHAPE), ("dk", 0, E_SHAPE),
    ("io", 7, E_DTYPE),
    ("decay", 3, E_ARGS), ("erase", 3, E_ARGS), ("write", -1, E_ARGS), ("qmix", 3, E_ARGS),
    ("erase", 2, E_ARGS), ("write", 2, E_ARGS),
    ("q", 0, E_NULL), ("o", 0, E_NULL), ("g", 0, E_NULL), ("beta", 0, E_NULL),
    ("q", _addr(0, 8), E_ALIGN), ("state_out", _addr(7, 4), E_ALIGN), ("beta", _addr(5, 2), E_ALIGN),
    ("dk", 96, E_UNSUP), ("dv", 40, E_UNSUP), ("dv_split", 48, E_UNSUP),
])
def test_single_bad_field(lib, field, value, code):
    a = good_args(**{field: value})
    assert _validate(lib, a) == code, lib.gdr_last_error()
    assert lib.gdr_last_error()  # a message is set


def test_error_paths_return_before_launch(lib):
    # the full entry points give the same codes without touching a device
    a = good_args(B=0)
    assert lib.gdr_chunk_fwd(ctypes.byref(a), None) == E_SHAPE
    a = good_args(T=5)
    assert lib.gdr_recurrent_step(ctypes.byref(a), None) == E_SHAPE
    a = good_args(io=1, dk=256, T=1)
    assert lib.gdr_recurrent_step(ctypes.byref(a), None) == E_UNSUP


def test_kind_consistency(lib):
    assert _validate(lib, good_args(decay=0)) == E_ARGS           # g given with decay NONE
    assert _validate(lib, good_args(decay=0, g=0)) == OK
    assert _validate(lib, good_args(qmix=1)) == E_NULL            # lambda missing
    assert _validate(lib, good_args(qmix=1, lambda_=_addr(8))) == OK
    assert _validate(lib, good_args(qmix=1, lambda_=_addr(8), erase=1, b=_addr(9))) == E_ARGS
    assert _validate(lib, good_args(erase=1)) == E_NULL           # b missing
    assert _validate(lib, good_args(erase=1, b=_addr(9))) == OK
    assert _validate(lib, good_args(write=1, beta=0)) == E_NULL   # erase still needs beta
    assert _validate(lib, good_args(write=1, erase=1, beta=0, b=_addr(9), w=_addr(10))) == OK
    assert _validate(lib, good_args(decay=2, g=_addr(4, 4))) == E_ALIGN  # channel g is vector-loaded


def test_time_varying_lambda_and_value_beta(lib):
    # lambda_t [B,T,H] and beta per value channel [B,T,H,dv] (erase = write = VALUE)
    assert _validate(lib, good_args(qmix=2, lambda_=_addr(8))) == OK
    assert _validate(lib, good_args(qmix=2, lambda_=0)) == E_NULL
    assert _validate(lib, good_args(erase=2, write=2)) == OK
    assert _validate(lib, good_args(erase=2, write=2, beta=0)) == E_NULL
    assert _validate(lib, good_args(erase=2, write=2, qmix=1, lambda_=_addr(8))) == E_ARGS
    # the aliasing check sizes beta [B,T,H,dv] and lambda [B,T,H]: o placed
    # just past [B,T,H] floats but inside the larger tensors is rejected
    tokens = 2 * 4 * 200
    assert _validate(lib, good_args(erase=2, write=2, o=_addr(5, tokens * 4 + 256))) == E_ARGS
    assert _validate(lib, good_args(o=_addr(5, tokens * 4 + 256))) == OK
    assert _validate(lib, good_args(qmix=2, lambda_=_addr(8), o=_addr(8, 4 * 4 + 256))) == E_ARGS
    assert _validate(lib, good_args(qmix=1, lambda_=_addr(8), o=_addr(8, 4 * 4 + 256))) == OK
    # both run on the plain fp32 kernel: 16-column slices, four waves
    for kw in (dict(qmix=2, lambda_=_addr(8)), dict(erase=2, write=2)):
        a = good_args(B=8, H=16, **kw)
        info = GdrPlanInfo()
        assert lib.gdr_plan(ctypes.byref(a), CHUNK, ctypes.byref(info)) == OK
        assert info.dv_slice == 16 and info.block == 256 and info.grid == 8 * 16 * 8
        assert _validate(lib, good_args(dv_split=32, **kw)) == E_UNSUP
        assert _validate(lib, good_args(T=1, **kw), STEP) == OK


def test_byte_offsets_fit_32_bits(lib):
    # a chunk's 64 rows of H * max(dk, dv) fp32 are addressed with 32-bit byte
    # offsets: H * max(dk, dv) must stay below 2^24
    # (gdr_plan: shape checks without the pointer checks, whose fake buffers
    # are too close together for these sizes)
    lim = (1 << 24) // 128
    info = GdrPlanInfo()
    for H, code in ((lim - 1, OK), (lim, E_SHAPE), (160000, E_SHAPE)):
        a = good_args(B=1, T=64, H=H)
        assert lib.gdr_plan(ctypes.byref(a), CHUNK, ctypes.byref(info)) == code, H


def test_aliasing(lib):
    assert _validate(lib, good_args(o=_addr(0))) == E_ARGS              # o on top of q
    assert _validate(lib, good_args(state_out=_addr(6))) == OK          # exact in-place state
    assert _validate(lib, good_args(state_out=_addr(6, 64))) == E_ARGS  # partial overlap
    assert _validate(lib, good_args(o=_addr(2, 16))) == E_ARGS          # inside v


def test_fp32_support_matrix(lib):
    assert _validate(lib, good_args(io=0, dk=64, dv=64)) == OK
    assert _validate(lib, good_args(io=0, dk=128)) == OK
    assert _validate(lib, good_args(io=0, dk=96)) == E_UNSUP
    assert _validate(lib, good_args(io=0, dk=64, dv=64, dv_split=64)) == E_UNSUP
    assert _validate(lib, good_args(io=0, dk=128, dv_split=32)) == E_UNSUP   # plain kernel: 16 columns
    assert _validate(lib, good_args(io=0, dk=128, T=1), STEP) == OK
    # fp32 at dk = 128 runs the plain fp32 kernel (16-column slices): one
    # pass without a workspace, the two-pass form (records once per chunk)
    # with one
    a = good_args(io=0, dk=128, B=1, H=2)
    info = GdrPlanInfo()
    assert lib.gdr_plan(ctypes.byref(a), CHUNK, ctypes.byref(info)) == OK
    assert info.dv_slice == 16 and info.block == 256 and info.passes == 1
    st, need = _ws_size(lib, a)
    assert st == OK and need == plain_record_bytes(1 * 2 * 4, 128)   # T = 200: 4 chunks
    a.workspace, a.workspace_bytes = _addr(11), need
    assert lib.gdr_plan(ctypes.byref(a), CHUNK, ctypes.byref(info)) == OK
    # the two-pass recurrence on the matrix cores: 64-column slices
    assert info.passes == 2 and info.dv_slice == 64 and info.block == 256
    assert info.grid == 2 * 2 and 0 < info.lds_bytes <= 160 * 1024
    # a caller's 16-column split, and the per-value-channel beta, keep the
    # vector-ALU recurrence (16 columns, two workgroups per CU)
    a.dv_split = 16
    assert lib.gdr_plan(ctypes.byref(a), CHUNK, ctypes.byref(info)) == OK
    assert info.passes == 2 and info.dv_slice == 16 and info.grid == 2 * 8
    assert 0 < info.lds_bytes <= 160 * 1024 // 2


def plain_record_bytes(nrec, dk):
    """Workspace of the plain kernel's two-pass form: T, A_qk [64][64],
    E_bar, Q_gamma, K_tail [64][dk], gamma_C [dk] fp32 per record, each
    array 256-byte aligned."""
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    return 2 * up(nrec * 64 * 64 * 4) + 3 * up(nrec * 64 * dk * 4) + up(nrec * dk * 4)


@pytest.mark.parametrize("B,H,T,dk,io", [(1, 2, 200, 128, 0), (2, 3, 65, 128, 0), (1, 1, 1, 128, 0)])
def test_plain_workspace_size(lib, B, H, T, dk, io):
    a = good_args(io=io, dk=dk, dv=64, B=B, H=H, T=T)
    st, n = _ws_size(lib, a)
    assert st == OK, lib.gdr_last_error()
    assert n == plain_record_bytes(B * H * ((T + 63) // 64), dk)


def test_zero_length_sequence_needs_no_token_pointers(lib):
    a = good_args(T=0, q=0, k=0, v=0, o=0, g=0, beta=0)
    assert _validate(lib, a) == OK


@pytest.mark.parametrize("B,H,dv,io,expect", [
    (8, 16, 128, 1, 64),   # 128 heads -> two 64-column slices -> 256 workgroups
    (8, 8, 128, 1, 32),    # 64 heads -> four slices
    (1, 32, 128, 1, 16),   # 32 heads -> eight slices
    (1, 2, 64, 0, 16),     # fp32, tiny: narrowest slice
])
def test_plan_slice_choice(lib, B, H, dv, io, expect):
    a = good_args(B=B, H=H, dv=dv, io=io, dk=64 if io == 0 else 128)
    info = GdrPlanInfo()
    assert lib.gdr_plan(ctypes.byref(a), CHUNK, ctypes.byref(info)) == OK
    assert info.dv_slice == expect
    assert info.grid == B * H * (dv // expect)
    # bf16 with scalar decay and the beta erase gate runs the pipelined kernel:
    # four producer waves plus two consumer waves (one for a 16-column slice)
    assert info.block == (64 * ((2 if expect >= 32 else 1) + 4) if io == 1 else 256)
    assert 0 < info.lds_bytes <= 160 * 1024
    assert info.n_chunks == (a.T + 63) // 64


@pytest.mark.parametrize("decay,erase,block", [(2, 0, 512), (2, 1, 512), (1, 1, 256), (0, 1, 256), (0, 0, 384),
                                               (1, 0, 384)])
def test_plan_kernel_choice(lib, decay, erase, block):
    """bf16 I/O runs a pipelined kernel (two consumer waves plus four producer
    waves, or six under a per-channel decay) except with the per-channel erase
    gate under no or a scalar decay, which runs the one-pass kernel (one
    256-thread workgroup)."""
    a = good_args(B=8, H=16, dv=128, decay=decay, erase=erase, **({"g": 0} if decay == 0 else {}))
    if erase == 1:
        a.b = a.beta
    info = GdrPlanInfo()
    assert lib.gdr_plan(ctypes.byref(a), CHUNK, ctypes.byref(info)) == OK
    assert info.block == block and info.dv_slice == 64


# ---- the workspace of the two-pass per-channel form ---------------------------

REC = 3 * 64 * 128 * 2 + 2 * 10 * 16 * 16 * 2 + 128 * 4  # one chunk's record (per-channel decay): 10 blocks of A, A_qk
REC_SCALAR = 11776                                   # 10 blocks of A, A_qk, 336 scalars, rounded to 256 (scalar decay)


def _chan_args(**kw):
    """Gated DeltaNet-2 kinds (per-channel decay, erase and write gates)."""
    base = dict(decay=2, erase=1, write=1, beta=0, b=_addr(9), w=_addr(10))
    base.update(kw)
    return good_args(**base)


def _ws_size(lib, a):
    n = ctypes.c_uint64(123)
    st = lib.gdr_workspace_size(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("B,H,T,dk,decay,erase,expect_chunks", [
    (1, 32, 200, 128, 2, 1, 4),   # 32 heads -> 16-column slices: two-pass form, 4 chunks each
    (2, 16, 65, 128, 2, 1, 2),    # 32 heads, ragged tail
    (2, 32, 200, 128, 2, 1, 4),   # 64 heads -> 32-column slices
    (8, 16, 200, 128, 2, 1, 0),   # 128 heads -> 64-column slices: single pass
    (1, 32, 200, 64, 2, 1, 0),    # dk 64: single pass
    (1, 32, 200, 128, 1, 0, 4),   # scalar decay: the scalar-decay form's smaller records
    (8, 8, 4096, 128, 1, 0, 64),  # the Q-Delta workload's shape
    (8, 16, 4096, 128, 1, 0, 0),  # the headline workload's shape: single pass
    (1, 32, 200, 128, 1, 1, 0),   # scalar decay, per-channel erase: the one-pass kernel
    (1, 32, 0, 128, 2, 1, 0),     # nothing to do
])
def test_workspace_size(lib, B, H, T, dk, decay, erase, expect_chunks):
    kw = {} if decay == 2 else dict(erase=erase, write=0, beta=_addr(5), b=_addr(9) if erase else 0, w=0)
    a = _chan_args(B=B, H=H, T=T, dk=dk, decay=decay, **kw)
    st, n = _ws_size(lib, a)
    assert st == OK, lib.gdr_last_error()
    assert n == B * H * expect_chunks * (REC if decay == 2 else REC_SCALAR)


def test_workspace_switches_the_plan(lib):
    a = _chan_args(B=1, H=32, T=200)
    st, need = _ws_size(lib, a)
    assert st == OK and need == 32 * 4 * REC
    info = GdrPlanInfo()
    assert lib.gdr_plan(ctypes.byref(a), CHUNK, ctypes.byref(info)) == OK
    assert info.passes == 1 and info.block == 64 * 7   # single pass: 1 consumer + 6 producer waves
    a.workspace, a.workspace_bytes = _addr(11), need - 1  # too small: still one pass
    assert lib.gdr_plan(ctypes.byref(a), CHUNK, ctypes.byref(info)) == OK and info.passes == 1
    a.workspace_bytes = need
    assert lib.gdr_plan(ctypes.byref(a), CHUNK, ctypes.byref(info)) == OK
    assert info.passes == 2 and info.dv_slice == 16 and info.grid == 32 * 8
    assert info.block == 64 * 5 and 0 < info.lds_bytes <= 160 * 1024   # 1 consumer + 4 loader waves


def test_noalloc_rejects_records_beyond_its_scratch(lib):
    # Gated DeltaNet-2 at B1 H32 T65536 needs 1.96 GB of records, far beyond
    # the 64 MiB scratch: rejected in host code, before any HIP call
    a = _chan_args(B=1, H=32, T=65536)
    st, need = _ws_size(lib, a)
    assert st == OK and need > (64 << 20)
    assert lib.gdr_chunk_fwd_noalloc(ctypes.byref(a), None) == E_SHAPE
    assert b"scratch" in lib.gdr_last_error()
    # the plain fp32 kernel falls back to its single pass instead (it needs
    # no records): the call gets past the host checks to the launch, which
    # fails here only for want of a GPU
    a = good_args(io=0, dk=128, B=8, H=16, T=4096)
    st, need = _ws_size(lib, a)
    assert st == OK and need > (64 << 20)
    assert lib.gdr_chunk_fwd_noalloc(ctypes.byref(a), None) not in (E_SHAPE, OK)
    assert b"scratch" not in lib.gdr_last_error()
    # validation errors come first, as for gdr_chunk_fwd
    a = good_args(B=0)
    assert lib.gdr_chunk_fwd_noalloc(ctypes.byref(a), None) == E_SHAPE
    assert lib.gdr_chunk_fwd_noalloc(None, None) == E_NULL


def test_version_one_struct_runs_without_workspace(lib):
    v1 = GdrArgs.workspace.offset
    a = _chan_args(B=1, H=32, T=200, workspace=_addr(11), workspace_bytes=1 << 40)
    a.struct_size = v1
    info = GdrPlanInfo()
    assert lib.gdr_plan(ctypes.byref(a), CHUNK, ctypes.byref(info)) == OK and info.passes == 1
    a.struct_size = v1 - 8
    assert _validate(lib, a) == E_ARGS


def test_workspace_errors_return_before_launch(lib):
    a = _chan_args(B=1, H=32, T=200)
    _, need = _ws_size(lib, a)
    a.workspace, a.workspace_bytes = _addr(11, 128), need      # not 256-byte aligned
    assert lib.gdr_chunk_fwd(ctypes.byref(a), None) == E_ALIGN
    a.workspace = _addr(0)                                      # on top of q
    assert lib.gdr_chunk_fwd(ctypes.byref(a), None) == E_ARGS
    assert b"workspace" in lib.gdr_last_error()
    n = ctypes.c_uint64(0)
    assert lib.gdr_workspace_size(None, ctypes.byref(n)) == E_NULL
    assert lib.gdr_workspace_size(ctypes.byref(a), None) == E_NULL


# ---- the recurrent form and the output epilogue -------------------------------

def test_recurrent_form_validation_and_plan(lib):
    assert _validate(lib, good_args(), RECUR) == OK
    assert _validate(lib, good_args(T=0, q=0, k=0, v=0, o=0, g=0, beta=0), RECUR) == OK
    assert _validate(lib, good_args(dk=96), RECUR) == E_UNSUP
    assert _validate(lib, good_args(dv=256), RECUR) == E_UNSUP
    assert _validate(lib, good_args(), 3) == E_ARGS
    info = GdrPlanInfo()
    a = good_args(B=4, H=8, dv=64)
    assert lib.gdr_plan(ctypes.byref(a), RECUR, ctypes.byref(info)) == OK
    assert info.grid == 32 and info.block == 64 and info.dv_slice == 64
    a = good_args(B=0)
    assert lib.gdr_recurrent_fwd(ctypes.byref(a), None) == E_SHAPE


def test_epilogue_fields(lib):
    fp = ctypes.POINTER(ctypes.c_float)
    def epi(**kw):
        a = good_args(**kw)
        a.out_gate = _addr(12)
        a.norm_weight = ctypes.cast(ctypes.c_void_p(_addr(13)), fp)
        return a
    for op in (CHUNK, STEP, RECUR):
        a = epi(T=1 if op == STEP else 200)
        assert _validate(lib, a, op) == OK, lib.gdr_last_error()
        a.norm_weight = fp()
        assert _validate(lib, a, op) == E_NULL
        a = epi(T=1 if op == STEP else 200)
        a.out_gate = _addr(12, 8)
        assert _validate(lib, a, op) == E_ALIGN
        a = epi(T=1 if op == STEP else 200, o=_addr(12, 64))       # o inside the gate
        assert _validate(lib, a, op) == E_ARGS
    assert _validate(lib, epi(dv=192, dv_split=64), CHUNK) == E_UNSUP   # the chunk epilogue: dv 64, 128, 256
    assert _validate(lib, good_args(dv=192, dv_split=64), CHUNK) == OK
    # a version-2 struct has no epilogue fields: they are not read
    a = epi()
    a.struct_size = GdrArgs.out_gate.offset
    a.norm_weight = fp()
    assert _validate(lib, a, CHUNK) == OK


def _norm(**kw):
    a = GdrNormArgs()
    a.struct_size = ctypes.sizeof(GdrNormArgs)
    a.dv, a.io, a.eps, a.rows = 128, 1, 0.0, 1000
    a.o, a.gate, a.y = _addr(0), _addr(1), _addr(2)
    a.weight = ctypes.cast(ctypes.c_void_p(_addr(3)), ctypes.POINTER(ctypes.c_float))
    for key, val in kw.items():
        setattr(a, key, val)
    return a


def test_output_norm_gate_errors_return_before_launch(lib):
    f = lib.gdr_output_norm_gate
    assert f(None, None) == E_NULL
    assert f(ctypes.byref(_norm(struct_size=8)), None) == E_ARGS
    assert f(ctypes.byref(_norm(io=5)), None) == E_DTYPE
    assert f(ctypes.byref(_norm(dv=96)), None) == E_UNSUP
    assert f(ctypes.byref(_norm(rows=-1)), None) == E_SHAPE
    assert f(ctypes.byref(_norm(rows=0, o=0, gate=0, y=0)), None) == OK
    assert f(ctypes.byref(_norm(gate=0)), None) == E_NULL
    assert f(ctypes.byref(_norm(y=_addr(2, 8))), None) == E_ALIGN
    assert f(ctypes.byref(_norm(y=_addr(0, 256))), None) == E_ARGS      # partial overlap with o
    assert f(ctypes.byref(_norm(y=_addr(1))), None) == E_ARGS           # y on the gate


# ---- the backward ---------------------------------------------------------------

def _bwd(lib, fwd, **kw):
    from gated_delta_rule_17_amd._lib import GdrBwdArgs
    fp = ctypes.POINTER(ctypes.c_float)
    a = GdrBwdArgs()
    a.struct_size = ctypes.sizeof(GdrBwdArgs)
    a.fwd = ctypes.pointer(fwd)
    a.d_o = _addr(20)
    for i, name in enumerate(("dq", "dk", "dv", "dg", "dbeta", "dstate")):
        setattr(a, name, ctypes.cast(ctypes.c_void_p(_addr(21 + i)), fp))
    a.workspace, a.workspace_bytes = _addr(40), 1 << 40
    for key, val in kw.items():
        if key in ("dq", "dk", "dv", "dg", "dbeta", "db", "dw", "dlam", "dstate", "d_state"):
            val = ctypes.cast(ctypes.c_void_p(val), fp) if val else fp()
        setattr(a, key, val)
    return a


def test_backward_workspace_and_validation(lib):
    from gated_delta_rule_17_amd._lib import GdrBwdArgs  # noqa: F401
    f = good_args(B=2, H=4, T=200, o=0)
    a = _bwd(lib, f)
    n = ctypes.c_uint64(0)
    assert lib.gdr_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n)) == OK, lib.gdr_last_error()
    # per chunk-head: S, dS (dk dv), W, dR (64 dv), T, A (64 x 64), E_bar, Q_gamma, K_tail (64 dk), gamma_C (dk)
    per = (2 * 128 * 128 + 2 * 64 * 128 + 2 * 64 * 64 + 3 * 64 * 128 + 128) * 4
    assert n.value == 2 * 4 * 4 * per
    f.erase = f.write = 2                       # per-value-channel beta: no backward
    assert lib.gdr_bwd_workspace_size(ctypes.byref(_bwd(lib, f)), ctypes.byref(n)) == E_UNSUP
    f = good_args(B=2, H=4, T=200, o=0, dk=96)
    assert lib.gdr_bwd_workspace_size(ctypes.byref(_bwd(lib, f)), ctypes.byref(n)) == E_UNSUP
    # error paths of gdr_chunk_bwd, all before any launch
    f = good_args(B=2, H=4, T=200, o=0)
    assert lib.gdr_chunk_bwd(None, None) == E_NULL
    assert lib.gdr_chunk_bwd(ctypes.byref(_bwd(lib, f, dg=0)), None) == E_NULL
    assert lib.gdr_chunk_bwd(ctypes.byref(_bwd(lib, f, workspace_bytes=16)), None) == E_ARGS
    assert lib.gdr_chunk_bwd(ctypes.byref(_bwd(lib, f, workspace=_addr(40, 64))), None) == E_ALIGN
    assert lib.gdr_chunk_bwd(ctypes.byref(_bwd(lib, f, dq=_addr(0))), None) == E_ARGS      # dq on q
    assert lib.gdr_chunk_bwd(ctypes.byref(_bwd(lib, f, dk=_addr(21, 128))), None) == E_ARGS  # dk inside dq
    f.qmix = 1
    f.lambda_ = ctypes.cast(ctypes.c_void_p(_addr(8)), ctypes.POINTER(ctypes.c_float))
    assert lib.gdr_chunk_bwd(ctypes.byref(_bwd(lib, f)), None) == E_NULL                   # dlam missing
