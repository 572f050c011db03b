"""ctypes declarations of the C ABI in include/muon_adamw.h.

Loading fails loudly when the shared library has not been built: there is no
fallback path of any kind.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MA_LIBRARY", os.path.join(HERE, "libmuon_adamw.so"))

MA_OK = 0
MA_ERR_INVALID_ARG = -1
MA_ERR_UNSUPPORTED = -2
MA_ERR_WORKSPACE = -3
MA_ERR_HIP = -4
MA_ERR_NONFINITE = -5

MA_F32 = 0
MA_BF16 = 1
MA_EQ_OFF, MA_EQ_ROWS_PRE, MA_EQ_ROWS_POST, MA_EQ_ROWS_RMS = 0, 1, 2, 3
MA_SCALE_NONE, MA_SCALE_SQRT_MAX1_R_OVER_C, MA_SCALE_MOONSHOT, MA_SCALE_SQRT_MAX = 0, 1, 2, 3
MA_MAX_NS_STEPS = 16
KERNEL_KINDS = ("rownorm", "finalize", "pre", "gram", "poly", "axpy", "post", "adamw", "lion", "axpy_update")
MA_WORKSPACE_ALIGN = 256
MA_NOALLOC_SCRATCH_BYTES = 64 << 20


class MuonGroupC(C.Structure):
    _fields_ = [
        ("rows", C.c_int64), ("cols", C.c_int64), ("count", C.c_int32),
        ("param_dtype", C.c_int32), ("grad_dtype", C.c_int32), ("mom_dtype", C.c_int32),
        ("params", C.POINTER(C.c_void_p)), ("grads", C.POINTER(C.c_void_p)),
        ("momentum", C.POINTER(C.c_void_p)),
    ]


class MuonHParamsC(C.Structure):
    _fields_ = [
        ("lr", C.c_float), ("momentum", C.c_float), ("weight_decay", C.c_float),
        ("nesterov", C.c_int32), ("ns_steps", C.c_int32), ("abc", C.POINTER(C.c_float)),
        ("cautious", C.c_int32), ("equilibrate", C.c_int32), ("ns_precision", C.c_int32),
        ("lr_scale", C.c_int32), ("norm_eps", C.c_float), ("eq_eps", C.c_float),
        ("check_finite", C.c_int32),
    ]


class AdamWSegmentC(C.Structure):
    _fields_ = [
        ("param", C.c_void_p), ("grad", C.c_void_p), ("exp_avg", C.c_void_p),
        ("exp_avg_sq", C.c_void_p), ("n", C.c_int64), ("param_dtype", C.c_int32),
        ("grad_dtype", C.c_int32), ("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float),
        ("eps", C.c_float), ("weight_decay", C.c_float), ("step", C.c_int64),
    ]


class LionSegmentC(C.Structure):
    _fields_ = [
        ("param", C.c_void_p), ("grad", C.c_void_p), ("exp_avg", C.c_void_p), ("n", C.c_int64),
        ("param_dtype", C.c_int32), ("grad_dtype", C.c_int32), ("lr", C.c_float), ("beta1", C.c_float),
        ("beta2", C.c_float), ("weight_decay", C.c_float),
    ]


EXPORTS = {
    "ma_muon_workspace_size": (C.c_size_t, [C.POINTER(MuonGroupC), C.c_int32, C.POINTER(MuonHParamsC)]),
    "ma_muon_step": (C.c_int, [C.POINTER(MuonGroupC), C.c_int32, C.POINTER(MuonHParamsC), C.c_void_p,
                               C.c_size_t, C.c_void_p]),
    "ma_muon_step_noalloc": (C.c_int, [C.POINTER(MuonGroupC), C.c_int32, C.POINTER(MuonHParamsC), C.c_void_p]),
    "ma_muon_step_stats": (C.c_int, [C.POINTER(MuonGroupC), C.c_int32, C.POINTER(MuonHParamsC), C.c_void_p,
                                     C.c_size_t, C.c_void_p, C.c_void_p]),
    "ma_muon_nonfinite": (C.c_int, [C.POINTER(MuonGroupC), C.c_int32, C.POINTER(MuonHParamsC), C.c_void_p,
                                    C.c_void_p]),
    "ma_muon_row_pass": (C.c_int, [C.POINTER(MuonGroupC), C.c_int32, C.POINTER(MuonHParamsC), C.c_int32]),
    "ma_muon_workspace_update": (C.c_int, [C.POINTER(MuonGroupC), C.c_int32, C.POINTER(MuonHParamsC),
                                           C.c_void_p, C.c_int32, C.c_int32, C.POINTER(C.c_void_p),
                                           C.POINTER(C.c_int64), C.POINTER(C.c_int32),
                                           C.POINTER(C.c_int32)]),
    "ma_adamw_step": (C.c_int, [C.POINTER(AdamWSegmentC), C.c_int32, C.c_void_p]),
    "ma_adamw_step_background": (C.c_int, [C.POINTER(AdamWSegmentC), C.c_int32, C.c_int32, C.c_void_p]),
    "ma_muon_adamw_step": (C.c_int, [C.POINTER(MuonGroupC), C.c_int32, C.POINTER(MuonHParamsC), C.c_void_p,
                                     C.c_size_t, C.POINTER(AdamWSegmentC), C.c_int32, C.c_int32, C.c_void_p,
                                     C.c_void_p]),
    "ma_lion_step": (C.c_int, [C.POINTER(LionSegmentC), C.c_int32, C.c_void_p]),
    "ma_status_string": (C.c_char_p, [C.c_int]),
    "ma_last_error": (C.c_char_p, []),
    "ma_version": (C.c_char_p, []),
    "ma_profile_begin": (C.c_int, [C.c_int32]),
    "ma_profile_end": (C.c_int, []),
    "ma_profile_read": (C.c_int, [C.c_int32, C.POINTER(C.c_double), C.POINTER(C.c_int64)]),
    "ma_calib_mfma": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
    "ma_test_bf16_round": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]),
    "ma_test_muon_momentum": (C.c_int, [C.POINTER(MuonGroupC), C.c_float, C.c_int32, C.c_void_p,
                                        C.c_void_p]),
    "ma_test_muon_update": (C.c_int, [C.POINTER(MuonGroupC), C.c_void_p, C.c_int32, C.c_float,
                                      C.c_float, C.c_int32, C.c_int32, C.c_void_p]),
    "ma_test_fail_after_fork": (C.c_int, []),
    "ma_test_ns_workspace_size": (C.c_size_t, [C.c_int64, C.c_int64, C.c_int32, C.c_int32]),
    "ma_test_ns": (C.c_int, [C.c_int64, C.c_int64, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                             C.POINTER(C.c_float), C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p]),
}

_lib = None


class MuonAdamWError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def lib() -> C.CDLL:
    """The loaded shared library (loaded once)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m adamw_optimizer_step_amd.build` "
                "(the Muon/AdamW step has no other implementation)")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def check(status: int) -> None:
    if status != MA_OK:
        msg = lib().ma_last_error().decode(errors="replace")
        raise MuonAdamWError(status, msg or lib().ma_status_string(status).decode())
