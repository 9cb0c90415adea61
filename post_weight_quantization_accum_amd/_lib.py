"""ctypes binding of libgptq_mi355x.so: argument marshalling only.

Every step of the solver runs in the HIP library.  This module turns torch
tensors into device pointers and sizes, passes the current HIP stream, and
turns non-OK status codes into exceptions.  If the shared library is missing
it raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgptq_mi355x.so")

# gptq_status
OK, ERR_INVALID_ARG, ERR_NOT_PD, ERR_NONFINITE, ERR_WORKSPACE, ERR_HIP, ERR_UNSUPPORTED = range(7)
# gptq_dtype
F32, F16, BF16 = 0, 1, 2

# Every symbol include/gptq.h declares.
EXPORTS = (
    "gptq_config_default", "gptq_hessian_workspace", "gptq_hessian_accumulate", "gptq_hessian_accumulate_timed",
    "gptq_hessian_accumulate_noalloc",
    "gptq_prepare_hinv_workspace", "gptq_prepare_hinv", "gptq_quantize_layer_workspace",
    "gptq_quantize_layer", "gptq_prepare_hinv_factored_workspace", "gptq_prepare_hinv_factored",
    "gptq_quantize_layer_factored_workspace", "gptq_quantize_layer_factored",
    "gptq_packed_words_per_row", "gptq_pack", "gptq_pack_permuted",
    "gptq_dequant_max_groups", "gptq_dequant_matmul", "gptq_gather_columns", "gptq_status_string",
    "gptq_version",
)


class GPTQError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


class NotPositiveDefinite(GPTQError):
    pass


class NonFinite(GPTQError):
    pass


class InvalidArgument(GPTQError):
    pass


class WorkspaceError(GPTQError):
    pass


class Unsupported(GPTQError):
    pass


_EXC = {ERR_INVALID_ARG: InvalidArgument, ERR_NOT_PD: NotPositiveDefinite, ERR_NONFINITE: NonFinite,
        ERR_WORKSPACE: WorkspaceError, ERR_UNSUPPORTED: Unsupported}


class Config(ctypes.Structure):
    """gptq_config."""
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32), ("sym", ctypes.c_int32),
                ("act_order", ctypes.c_int32), ("block_size", ctypes.c_int32), ("static_groups", ctypes.c_int32),
                ("damp", ctypes.c_double)]


def make_config(bits=4, group_size=128, sym=False, act_order=False, block=128, damp=0.01,
                static_groups=False) -> Config:
    return Config(int(bits), int(group_size), int(bool(sym)), int(bool(act_order)), int(block),
                  int(bool(static_groups)), float(damp))


_lib = None


def load(path: str | None = None):
    """Load the shared library (once).  Raises OSError when it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"{p} is missing: build it with `python -m post_weight_quantization_accum_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(Config)
    lib.gptq_config_default.argtypes = [cfgp]
    lib.gptq_config_default.restype = None
    lib.gptq_status_string.argtypes = [ctypes.c_int]
    lib.gptq_status_string.restype = ctypes.c_char_p
    lib.gptq_version.argtypes = []
    lib.gptq_version.restype = ctypes.c_char_p
    lib.gptq_hessian_workspace.argtypes = [i64, i64]
    lib.gptq_hessian_workspace.restype = sz
    lib.gptq_hessian_accumulate.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, vp, sz, vp]
    lib.gptq_hessian_accumulate.restype = ctypes.c_int
    lib.gptq_hessian_accumulate_timed.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, vp, sz, vp,
                                                  ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    lib.gptq_hessian_accumulate_timed.restype = ctypes.c_int
    lib.gptq_hessian_accumulate_noalloc.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, vp]
    lib.gptq_hessian_accumulate_noalloc.restype = ctypes.c_int
    lib.gptq_prepare_hinv_workspace.argtypes = [i64]
    lib.gptq_prepare_hinv_workspace.restype = sz
    lib.gptq_prepare_hinv.argtypes = [vp, i64, cfgp, vp, vp, sz, vp]
    lib.gptq_prepare_hinv.restype = ctypes.c_int
    lib.gptq_quantize_layer_workspace.argtypes = [i64, i64, cfgp]
    lib.gptq_quantize_layer_workspace.restype = sz
    lib.gptq_quantize_layer.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, cfgp, vp, vp, vp, vp, vp, vp,
                                        vp, sz, vp]
    lib.gptq_quantize_layer.restype = ctypes.c_int
    lib.gptq_prepare_hinv_factored_workspace.argtypes = [i64]
    lib.gptq_prepare_hinv_factored_workspace.restype = sz
    lib.gptq_prepare_hinv_factored.argtypes = [vp, i64, cfgp, vp, vp, sz, vp]
    lib.gptq_prepare_hinv_factored.restype = ctypes.c_int
    lib.gptq_quantize_layer_factored_workspace.argtypes = [i64, i64, cfgp]
    lib.gptq_quantize_layer_factored_workspace.restype = sz
    lib.gptq_quantize_layer_factored.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, cfgp, vp, vp, vp, vp, vp,
                                                 vp, vp, sz, vp]
    lib.gptq_quantize_layer_factored.restype = ctypes.c_int
    lib.gptq_packed_words_per_row.argtypes = [i64, i32]
    lib.gptq_packed_words_per_row.restype = i64
    lib.gptq_pack.argtypes = [vp, i64, i64, i32, vp, vp]
    lib.gptq_pack.restype = ctypes.c_int
    lib.gptq_pack_permuted.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    lib.gptq_pack_permuted.restype = ctypes.c_int
    lib.gptq_dequant_max_groups.argtypes = []
    lib.gptq_dequant_max_groups.restype = i64
    lib.gptq_dequant_matmul.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, i32, vp, vp, i64, vp, vp, i32, i64,
                                        vp, i64, vp]
    lib.gptq_dequant_matmul.restype = ctypes.c_int
    lib.gptq_gather_columns.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, i64, vp]
    lib.gptq_gather_columns.restype = ctypes.c_int
    _lib = lib
    return lib


def check(status: int, where: str):
    if status != OK:
        msg = load().gptq_status_string(status).decode()
        raise _EXC.get(status, GPTQError)(status, where, msg)


def status_string(status: int) -> str:
    return load().gptq_status_string(status).decode()


def version() -> str:
    return load().gptq_version().decode()
