"""ctypes loader for libgdr.so and the C structs of include/gdr.h."""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDR_LIBRARY selects another build of the library (e.g. the sanitized one)
_LIB_PATH = os.environ.get("GDR_LIBRARY") or os.path.join(_HERE, "libgdr.so")

EXPORTS = ["gdr_abi_version", "gdr_bwd_workspace_size", "gdr_chunk_bwd", "gdr_chunk_fwd", "gdr_chunk_fwd_noalloc", "gdr_last_error", "gdr_output_norm_gate",
           "gdr_plan", "gdr_recurrent_fwd", "gdr_recurrent_step", "gdr_status_str", "gdr_validate",
           "gdr_workspace_size"]

STATUS = {0: "GDR_OK", 1: "GDR_E_NULL", 2: "GDR_E_SHAPE", 3: "GDR_E_DTYPE", 4: "GDR_E_ALIGN",
          5: "GDR_E_UNSUPPORTED", 6: "GDR_E_HIP", 7: "GDR_E_ARGS"}

_FP = ctypes.POINTER(ctypes.c_float)


class GdrArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
        ("chunk", ctypes.c_int32), ("io", ctypes.c_int32), ("decay", ctypes.c_int32),
        ("erase", ctypes.c_int32), ("write", ctypes.c_int32), ("qmix", ctypes.c_int32),
        ("dv_split", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", _FP), ("beta", _FP), ("b", _FP), ("w", _FP), ("lambda_", _FP),
        ("state_in", _FP), ("state_out", _FP),
        ("o", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64),
        ("out_gate", ctypes.c_void_p), ("norm_weight", _FP), ("norm_eps", ctypes.c_float),
    ]


class GdrBwdArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("fwd", ctypes.POINTER(GdrArgs)),
                ("d_o", ctypes.c_void_p), ("d_state", _FP),
                ("dq", _FP), ("dk", _FP), ("dv", _FP), ("dg", _FP), ("dbeta", _FP), ("db", _FP), ("dw", _FP),
                ("dlam", _FP), ("dstate", _FP),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64)]


class GdrNormArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dv", ctypes.c_int32), ("io", ctypes.c_int32),
                ("eps", ctypes.c_float), ("rows", ctypes.c_int64),
                ("o", ctypes.c_void_p), ("gate", ctypes.c_void_p), ("weight", _FP), ("y", ctypes.c_void_p)]


class GdrPlanInfo(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_int32), ("block", ctypes.c_int32), ("dv_slice", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("n_chunks", ctypes.c_int32), ("passes", ctypes.c_int32)]


class GdrError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


_lib = None


def path() -> str:
    return _LIB_PATH


def load():
    """Load libgdr.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python gated_delta_rule_17_amd/csrc/build.py` (or __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.gdr_chunk_bwd.argtypes = [ctypes.POINTER(GdrBwdArgs), ctypes.c_void_p]
    lib.gdr_chunk_bwd.restype = ctypes.c_int
    lib.gdr_bwd_workspace_size.argtypes = [ctypes.POINTER(GdrBwdArgs), ctypes.POINTER(ctypes.c_uint64)]
    lib.gdr_bwd_workspace_size.restype = ctypes.c_int
    lib.gdr_output_norm_gate.argtypes = [ctypes.POINTER(GdrNormArgs), ctypes.c_void_p]
    lib.gdr_output_norm_gate.restype = ctypes.c_int
    for name in ("gdr_chunk_fwd", "gdr_chunk_fwd_noalloc", "gdr_recurrent_step", "gdr_recurrent_fwd"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.POINTER(GdrArgs), ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.gdr_validate.argtypes = [ctypes.POINTER(GdrArgs), ctypes.c_int]
    lib.gdr_validate.restype = ctypes.c_int
    lib.gdr_plan.argtypes = [ctypes.POINTER(GdrArgs), ctypes.c_int, ctypes.POINTER(GdrPlanInfo)]
    lib.gdr_plan.restype = ctypes.c_int
    lib.gdr_workspace_size.argtypes = [ctypes.POINTER(GdrArgs), ctypes.POINTER(ctypes.c_uint64)]
    lib.gdr_workspace_size.restype = ctypes.c_int
    lib.gdr_status_str.argtypes = [ctypes.c_int]
    lib.gdr_status_str.restype = ctypes.c_char_p
    lib.gdr_last_error.argtypes = []
    lib.gdr_last_error.restype = ctypes.c_char_p
    lib.gdr_abi_version.argtypes = []
    lib.gdr_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def call(name, args, *rest):
    lib = load()
    st = getattr(lib, name)(ctypes.byref(args), *rest)
    if st != 0:
        raise GdrError(st, lib.gdr_last_error().decode())
    return st
