"""ctypes view of ``include/dmuon.h`` and the loader of ``libdmuon.so``.

Argument marshalling only; every step of the computation runs in the HIP
library.  A missing library is an error, never a fallback.
"""

from __future__ import annotations

import ctypes
import os

# DMUON_LIB names another build of the same library (for instance the one
# with sanitized host code); by default the one built next to this file
LIB_PATH = os.environ.get("DMUON_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                       "libdmuon.so")

ABI_VERSION = 1

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED_DTYPE = -2
ERR_ALIAS = -3
ERR_WORKSPACE_TOO_SMALL = -4
ERR_MISALIGNED = -5
ERR_HIP = -6

BF16 = 0
F32 = 1
FIELD_PARAM = 0
FIELD_GRAD = 1
FLAG_NS_FP32 = 1 << 0
FLAG_NESTEROV = 1 << 1
FLAG_GRAM_NS = 1 << 2
FLAG_CHECK_FINITE = 1 << 3
FLAG_CHAIN_LAUNCH = 1 << 4

# dmuon_launch_info.kind
LAUNCH_KINDS = ("momentum_sumsq", "momentum_orient", "norm", "update_direct", "gram", "square",
                "apply", "final", "gram_square", "chain")

EXPORTED = ("dmuon_abi_version", "dmuon_error_string", "dmuon_last_error",
            "dmuon_partition_lpt", "dmuon_pack_offsets", "dmuon_workspace_bytes",
            "dmuon_pack", "dmuon_unpack", "dmuon_muon_step", "dmuon_muon_step_traced",
            "dmuon_muon_step_packed", "dmuon_adamw_step", "dmuon_step_launches",
            "dmuon_nonfinite_flags_offset", "dmuon_muon_step_noalloc",
            "dmuon_chain_status_offset")

# DMUON_NOALLOC_SCRATCH_BYTES
NOALLOC_SCRATCH_BYTES = 64 << 20


class Matrix(ctypes.Structure):
    """``dmuon_matrix``"""
    _fields_ = [
        ("param", ctypes.c_void_p),
        ("param_dtype", ctypes.c_int32),
        ("grad_dtype", ctypes.c_int32),
        ("grad", ctypes.c_void_p),
        ("momentum", ctypes.c_void_p),
        ("orth_out", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("reserved", ctypes.c_int32),
        ("packed_offset", ctypes.c_int64),
    ]


class StepConfig(ctypes.Structure):
    """``dmuon_step_config``"""
    _fields_ = [
        ("a", ctypes.c_float), ("b", ctypes.c_float), ("c", ctypes.c_float),
        ("ns_steps", ctypes.c_int32),
        ("lr", ctypes.c_float), ("momentum", ctypes.c_float), ("eps", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]


class LaunchInfo(ctypes.Structure):
    """``dmuon_launch_info``"""
    _fields_ = [("kind", ctypes.c_int32), ("tile", ctypes.c_int32), ("flops", ctypes.c_double)]


class Tensor(ctypes.Structure):
    """``dmuon_tensor``"""
    _fields_ = [
        ("param", ctypes.c_void_p),
        ("param_dtype", ctypes.c_int32),
        ("grad_dtype", ctypes.c_int32),
        ("grad", ctypes.c_void_p),
        ("exp_avg", ctypes.c_void_p),
        ("exp_avg_sq", ctypes.c_void_p),
        ("numel", ctypes.c_int64),
    ]


class AdamWConfig(ctypes.Structure):
    """``dmuon_adamw_config``"""
    _fields_ = [
        ("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int32),
    ]


class DmuonError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"dmuon status {status}: {message}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads the HIP library once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m newton_schulz_dmuon_amd.build`")
    try:
        # torch ships its own HIP runtime under the same soname; load it first
        # so this library binds to that one instead of a second copy
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    c_i32, c_i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    P = ctypes.POINTER
    lib.dmuon_abi_version.restype = ctypes.c_int
    lib.dmuon_error_string.restype = ctypes.c_char_p
    lib.dmuon_error_string.argtypes = [ctypes.c_int]
    lib.dmuon_last_error.restype = ctypes.c_char_p
    lib.dmuon_partition_lpt.argtypes = [P(c_i64), c_i32, c_i32, P(c_i32), P(c_i64)]
    lib.dmuon_pack_offsets.argtypes = [P(c_i64), c_i32, c_i64, P(c_i64), P(c_i64)]
    lib.dmuon_workspace_bytes.argtypes = [P(Matrix), c_i32, P(StepConfig), P(ctypes.c_size_t)]
    lib.dmuon_pack.argtypes = [P(Matrix), c_i32, c_i32, vp, c_i32, c_i64, vp]
    lib.dmuon_unpack.argtypes = [P(Matrix), c_i32, c_i32, vp, c_i32, c_i64, vp]
    lib.dmuon_muon_step.argtypes = [P(Matrix), c_i32, P(StepConfig), vp, ctypes.c_size_t, vp]
    lib.dmuon_muon_step_traced.argtypes = [P(Matrix), c_i32, P(StepConfig), vp,
                                           ctypes.c_size_t, vp, P(vp), c_i32]
    lib.dmuon_muon_step_packed.argtypes = [P(Matrix), c_i32, P(StepConfig), vp, ctypes.c_size_t,
                                           vp, c_i32, c_i64, vp, P(vp), c_i32]
    lib.dmuon_adamw_step.argtypes = [P(Tensor), c_i32, P(AdamWConfig), vp]
    lib.dmuon_step_launches.argtypes = [P(Matrix), c_i32, P(StepConfig), P(LaunchInfo), c_i32,
                                        P(c_i32)]
    lib.dmuon_nonfinite_flags_offset.argtypes = [P(Matrix), c_i32, P(StepConfig), P(ctypes.c_size_t)]
    lib.dmuon_chain_status_offset.argtypes = [P(Matrix), c_i32, P(StepConfig), P(ctypes.c_size_t)]
    lib.dmuon_muon_step_noalloc.argtypes = [P(Matrix), c_i32, P(StepConfig), vp]
    for name in ("dmuon_partition_lpt", "dmuon_pack_offsets", "dmuon_workspace_bytes",
                 "dmuon_pack", "dmuon_unpack", "dmuon_muon_step", "dmuon_muon_step_traced",
                 "dmuon_muon_step_packed", "dmuon_adamw_step", "dmuon_step_launches",
                 "dmuon_nonfinite_flags_offset", "dmuon_muon_step_noalloc",
                 "dmuon_chain_status_offset"):
        getattr(lib, name).restype = ctypes.c_int
    if lib.dmuon_abi_version() != ABI_VERSION:
        raise ImportError(f"libdmuon ABI {lib.dmuon_abi_version()} != {ABI_VERSION}")
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != OK:
        lib = load()
        raise DmuonError(status, f"{lib.dmuon_error_string(status).decode()}: "
                                 f"{lib.dmuon_last_error().decode()}")
