"""ctypes loader for libdmuon.so (the gfx950 HIP library built in-tree).

There is no fallback: if the library is missing or fails to load, every entry
point raises.  torch is imported first so that the library binds to the same
HIP runtime instance torch uses (both name it libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads torch's HIP runtime before ours)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdmuon.so")

DMUON_F32 = 0
DMUON_BF16 = 1

DMUON_OK = 0
DMUON_ERR_INVALID_ARG = 1
DMUON_ERR_UNSUPPORTED_DTYPE = 2
DMUON_ERR_WORKSPACE = 3
DMUON_ERR_NO_DEVICE = 4
DMUON_ERR_UNSUPPORTED_ARCH = 5
DMUON_ERR_HIP = 6

DMUON_MIN_NS_NUMEL = 100000
DMUON_MAX_DIM = 65536
DMUON_MAX_NS_STEPS = 64
DMUON_NOALLOC_SCRATCH_BYTES = 67108864

DMUON_NS_GRAM = 0
DMUON_NS_DIRECT = 1
DMUON_MAX_NS_TERMS = 3
DMUON_LR_SCALE_ONE = 0
DMUON_LR_SCALE_MOONLIGHT = 1


class NsConfig(ctypes.Structure):
    """dmuon_ns_config."""
    _fields_ = [
        ("backend", ctypes.c_int),
        ("num_terms", ctypes.c_int),
        ("per_step", ctypes.c_int),
        ("coeffs", ctypes.POINTER(ctypes.c_float)),
    ]


class KernelStat(ctypes.Structure):
    _fields_ = [
        ("name", ctypes.c_char * 40),
        ("launches", ctypes.c_int64),
        ("total_ms", ctypes.c_double),
        ("flops", ctypes.c_double),
        ("bytes", ctypes.c_double),
    ]


_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)
_I64P = ctypes.POINTER(ctypes.c_int64)
_SZP = ctypes.POINTER(ctypes.c_size_t)
_FP = ctypes.POINTER(ctypes.c_float)
_CFGP = ctypes.POINTER(NsConfig)

# name -> (restype, argtypes); mirrors include/dmuon.h
SIGNATURES = {
    "dmuon_ns_workspace_bytes": (ctypes.c_int, [ctypes.c_int, _I64P, _I64P, ctypes.c_int, _CFGP, _SZP]),
    "dmuon_ns_batched": (ctypes.c_int, [ctypes.c_int, _PP, _PP, _I64P, _I64P, ctypes.c_int, ctypes.c_int,
                                        _CFGP, _P, ctypes.c_size_t, _P]),
    "dmuon_muon_step_workspace_bytes": (ctypes.c_int, [ctypes.c_int, _I64P, _I64P, ctypes.c_int, _CFGP, _SZP]),
    "dmuon_muon_step": (ctypes.c_int, [ctypes.c_int, _PP, _PP, _PP, _I64P, _I64P, ctypes.c_int, ctypes.c_int,
                                       _CFGP, ctypes.c_float, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_int, _FP, _PP, _P, _P, ctypes.c_size_t, _P]),
    "dmuon_muon_step_clip_workspace_bytes": (ctypes.c_int, [ctypes.c_int, _I64P, _I64P, ctypes.c_int, _CFGP,
                                                            ctypes.c_int, _SZP]),
    "dmuon_muon_step_clipped": (ctypes.c_int, [ctypes.c_int, _PP, _PP, _PP, _I64P, _I64P, ctypes.c_int, ctypes.c_int,
                                               _CFGP, ctypes.c_float, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                               ctypes.c_int, _FP, _PP, _P, ctypes.POINTER(ctypes.c_int), ctypes.c_int,
                                               _FP, ctypes.c_float, _P, _P, ctypes.c_size_t, _P]),
    "dmuon_muon_step_noalloc": (ctypes.c_int, [ctypes.c_int, _PP, _PP, _PP, _I64P, _I64P, ctypes.c_int, ctypes.c_int,
                                               _CFGP, ctypes.c_float, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                               ctypes.c_int, _FP, _PP, _P, _P]),
    "dmuon_clip_grad_norm_workspace_bytes": (ctypes.c_int, [ctypes.c_int, _I64P, ctypes.c_int, _SZP]),
    "dmuon_clip_grad_norm": (ctypes.c_int, [ctypes.c_int, _PP, _I64P, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                            ctypes.c_int, _FP, ctypes.c_float, _P, _P, ctypes.c_size_t, _P]),
    "dmuon_adamw_step_workspace_bytes": (ctypes.c_int, [ctypes.c_int, _I64P, _SZP]),
    "dmuon_adamw_step": (ctypes.c_int, [ctypes.c_int, _PP, _PP, _PP, _PP, _I64P, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                        ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "dmuon_plan_summary": (ctypes.c_int, [ctypes.c_int, _I64P, _I64P, ctypes.c_int, _CFGP, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_char_p, ctypes.c_size_t, _SZP]),
    "dmuon_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dmuon_last_error": (ctypes.c_char_p, []),
    "dmuon_backend_info": (ctypes.c_char_p, []),
    "dmuon_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "dmuon_profile_read": (ctypes.c_int, [ctypes.POINTER(KernelStat), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]),
}

_lib = None


class DmuonError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status}){': ' + detail if detail else ''}")


def load() -> ctypes.CDLL:
    """Load libdmuon.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m newton_schulz_08_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().dmuon_status_string(int(status)).decode()


def last_error() -> str:
    return load().dmuon_last_error().decode()


def check(status: int, where: str) -> None:
    if status != DMUON_OK:
        raise DmuonError(status, where, last_error())
