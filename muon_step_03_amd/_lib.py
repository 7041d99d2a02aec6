"""ctypes declarations of libmuon.so (include/muon.h).  Loaded on first use.

There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmuon.so")

MUON_OK = 0
MUON_ERR_INVALID_ARGUMENT = 1
MUON_ERR_INVALID_SHAPE = 2
MUON_ERR_UNSUPPORTED_DTYPE = 3
MUON_ERR_WORKSPACE_TOO_SMALL = 4
MUON_ERR_HIP = 5

MUON_DTYPE_F32 = 0
MUON_DTYPE_BF16 = 1
MUON_VARIANT_MUON = 0
MUON_VARIANT_MUONGS = 1
MUON_VARIANT_MUONH = 2
MUON_VARIANT_NORMUON = 3
MUON_VARIANT_MEQMUON = 4
MUON_SCALE_KELLER = 0x100
MUON_STATS_PER_MATRIX = 5
MUON_MAX_DIM = 32768
MUON_MAX_NS_STEPS = 100
MUON_GROUPS_PER_LAUNCH = 8
MUON_ADAMW_MAX_ELEMENTS = 1 << 40
MUON_ADAMW_TENSORS_PER_LAUNCH = 32
MUON_NOALLOC_WORKSPACE_BYTES = 64 << 20

# Every symbol include/muon.h declares.
EXPORTS = (
    "muon_workspace_bytes", "muon_workspace_bytes_grouped", "muon_step",
    "muon_step_batched", "muon_step_grouped", "muon_status_string", "muon_last_hip_error",
    "muon_profile_enable", "muon_profile_read", "muon_phase_name",
    "muon_adamw_step", "muon_adamw_step_grouped", "muon_step_grouped_noalloc",
)
MUON_NUM_PHASES = 10


class MuonGroup(ctypes.Structure):
    _fields_ = [
        ("count", ctypes.c_int64),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("W_table", ctypes.c_void_p),
        ("G_table", ctypes.c_void_p),
        ("M_table", ctypes.c_void_p),
        ("W", ctypes.c_void_p),
        ("G", ctypes.c_void_p),
        ("M", ctypes.c_void_p),
    ]


class AdamwTensor(ctypes.Structure):
    _fields_ = [
        ("P", ctypes.c_void_p),
        ("G", ctypes.c_void_p),
        ("m", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("n", ctypes.c_int64),
        ("lr", ctypes.c_double),
        ("weight_decay", ctypes.c_double),
    ]


_lib = None

_STEP_SCALARS = [ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_int,
                 ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_int,
                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]


def lib():
    """The loaded library; raises RuntimeError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m muon_step_03_amd.build` "
            "(or __graft_entry__.build()); the Muon step has no non-HIP implementation")
    L = ctypes.CDLL(LIB_PATH)
    L.muon_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    L.muon_workspace_bytes.restype = ctypes.c_size_t
    L.muon_workspace_bytes_grouped.argtypes = [ctypes.POINTER(MuonGroup), ctypes.c_int, ctypes.c_int]
    L.muon_workspace_bytes_grouped.restype = ctypes.c_size_t
    L.muon_step.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                            ctypes.c_int64, ctypes.c_int64] + _STEP_SCALARS
    L.muon_step.restype = ctypes.c_int
    L.muon_step_batched.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_int64] + _STEP_SCALARS
    L.muon_step_batched.restype = ctypes.c_int
    L.muon_step_grouped.argtypes = [ctypes.POINTER(MuonGroup), ctypes.c_int] + _STEP_SCALARS
    L.muon_step_grouped.restype = ctypes.c_int
    L.muon_step_grouped_noalloc.argtypes = ([ctypes.POINTER(MuonGroup), ctypes.c_int]
                                            + _STEP_SCALARS[:9] + [ctypes.c_void_p, ctypes.c_void_p])
    L.muon_step_grouped_noalloc.restype = ctypes.c_int
    L.muon_status_string.argtypes = [ctypes.c_int]
    L.muon_status_string.restype = ctypes.c_char_p
    L.muon_last_hip_error.argtypes = []
    L.muon_last_hip_error.restype = ctypes.c_int
    L.muon_profile_enable.argtypes = [ctypes.c_int]
    L.muon_profile_enable.restype = ctypes.c_int
    L.muon_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                    ctypes.c_int]
    L.muon_profile_read.restype = ctypes.c_int
    L.muon_adamw_step.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                  ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                  ctypes.c_double, ctypes.c_int64, ctypes.c_void_p]
    L.muon_adamw_step.restype = ctypes.c_int
    L.muon_adamw_step_grouped.argtypes = [ctypes.POINTER(AdamwTensor), ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                          ctypes.c_int64, ctypes.c_void_p]
    L.muon_adamw_step_grouped.restype = ctypes.c_int
    L.muon_phase_name.argtypes = [ctypes.c_int]
    L.muon_phase_name.restype = ctypes.c_char_p
    _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().muon_status_string(int(status)).decode()
