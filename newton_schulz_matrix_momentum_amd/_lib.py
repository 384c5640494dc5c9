"""ctypes binding of libmuon's C ABI (include/muon.h).

Argument marshalling only: torch tensors are turned into device pointers and
the current HIP stream; every step of the optimizer runs in libmuon's kernels.
There is no fallback: if libmuon.so is missing or cannot be loaded, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; another build (a tuning variant) is loaded only by an
# explicit load(path) call, never through the environment
LIB_PATH = os.path.join(_PKG, "libmuon.so")

MUON_OK = 0
MUON_ERR_INVALID_ARG = 1
MUON_ERR_UNSUPPORTED = 2
MUON_ERR_WORKSPACE_TOO_SMALL = 3
MUON_ERR_HIP = 4

MUON_F32, MUON_F16, MUON_BF16 = 0, 1, 2
MUON_NS_DIRECT, MUON_NS_GRAM, MUON_LIMUON = 0, 1, 2

# every entry point declared in include/muon.h
EXPORTS = ("muon_options_init", "muon_workspace_size", "muon_step", "muon_step_static", "muon_adamw_step",
           "muon_debug_square_buffer", "muon_status_string", "muon_last_error", "muon_version")
# bytes of the static workspace of muon_step_static (MUON_STATIC_WORKSPACE_BYTES)
STATIC_WORKSPACE_BYTES = 64 << 20


class MuonParam(ctypes.Structure):
    _fields_ = [
        ("weight", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("momentum", ctypes.c_void_p),
        ("accel", ctypes.c_void_p),
        ("prev_grad", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("gamma", ctypes.c_float),
        ("ortho_out", ctypes.c_void_p),
        ("mona_lite", ctypes.c_void_p),
    ]


class MuonTrace(ctypes.Structure):
    _fields_ = [
        ("events", ctypes.POINTER(ctypes.c_void_p)),
        ("stages", ctypes.POINTER(ctypes.c_int32)),
        ("work", ctypes.POINTER(ctypes.c_double)),
        ("capacity", ctypes.c_int32),
        ("count", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("launches", ctypes.POINTER(ctypes.c_int32)),
    ]


MUON_STAGE_E1, MUON_STAGE_NORM, MUON_STAGE_E2, MUON_STAGE_GEMM, MUON_STAGE_E3, MUON_STAGE_ADAMW, \
    MUON_STAGE_SMALL = range(7)
STAGE_NAMES = {0: "e1", 1: "norm", 2: "e2", 3: "gemm", 4: "e3", 5: "adamw", 6: "small"}


class MuonOptions(ctypes.Structure):
    _fields_ = [
        ("grad_dtype", ctypes.c_int),
        ("ns_dtype", ctypes.c_int),
        ("coeffs", ctypes.POINTER(ctypes.c_float)),
        ("divisor", ctypes.c_float),
        ("restart_every", ctypes.c_int32),
        ("step", ctypes.c_int64),
        ("trace", ctypes.POINTER(MuonTrace)),
        ("sketch", ctypes.c_void_p),
        ("sketch_ld", ctypes.c_int64),
        ("rank", ctypes.c_int32),
        ("oversample", ctypes.c_int32),
        ("power_iters", ctypes.c_int32),
        ("rcond", ctypes.c_float),
    ]


class MuonAdamwParam(ctypes.Structure):
    _fields_ = [
        ("param", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("exp_avg", ctypes.c_void_p),
        ("exp_avg_sq", ctypes.c_void_p),
        ("numel", ctypes.c_int64),
    ]


class MuonError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("libmuon: %s (status %d)" % (message, status))
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libmuon.so and declare its signatures (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch's HIP runtime must be the process's only one: libmuon binds to the
    # libamdhip64.so.7 already loaded by torch (same SONAME), so that stream
    # and event handles from torch are valid inside libmuon.
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise MuonError(-1, "%s not found: build it with newton_schulz_matrix_momentum_amd.build.build()" % path)
    lib = ctypes.CDLL(path)
    lib.muon_options_init.argtypes = [ctypes.POINTER(MuonOptions)]
    lib.muon_options_init.restype = None
    lib.muon_workspace_size.argtypes = [ctypes.POINTER(MuonParam), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.POINTER(MuonOptions)]
    lib.muon_workspace_size.restype = ctypes.c_size_t
    lib.muon_step.argtypes = [ctypes.POINTER(MuonParam), ctypes.c_int,
                              ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                              ctypes.c_int, ctypes.c_int, ctypes.POINTER(MuonOptions),
                              ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.muon_step.restype = ctypes.c_int
    lib.muon_step_static.argtypes = [ctypes.POINTER(MuonParam), ctypes.c_int,
                                     ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                     ctypes.c_int, ctypes.c_int, ctypes.POINTER(MuonOptions), ctypes.c_void_p]
    lib.muon_step_static.restype = ctypes.c_int
    lib.muon_adamw_step.argtypes = [ctypes.POINTER(MuonAdamwParam), ctypes.c_int, ctypes.c_int,
                                    ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                    ctypes.c_int64, ctypes.POINTER(MuonTrace), ctypes.c_void_p]
    lib.muon_adamw_step.restype = ctypes.c_int
    lib.muon_debug_square_buffer.argtypes = [ctypes.POINTER(MuonParam), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.POINTER(MuonOptions), ctypes.c_int, ctypes.c_int,
                                             ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_int64),
                                             ctypes.POINTER(ctypes.c_int64)]
    lib.muon_debug_square_buffer.restype = ctypes.c_int
    lib.muon_status_string.argtypes = [ctypes.c_int]
    lib.muon_status_string.restype = ctypes.c_char_p
    lib.muon_last_error.argtypes = []
    lib.muon_last_error.restype = ctypes.c_char_p
    lib.muon_version.argtypes = []
    lib.muon_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return load().muon_last_error().decode()


def version() -> str:
    return load().muon_version().decode()


def check(status: int):
    if status != MUON_OK:
        lib = load()
        raise MuonError(status, "%s: %s" % (lib.muon_status_string(status).decode(), lib.muon_last_error().decode()))
