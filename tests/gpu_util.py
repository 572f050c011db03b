"""Helpers shared by the GPU tests (no optimizer arithmetic here)."""
import os
import sys

import numpy as np
import pytest
import torch

F32 = np.float32


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from adamw_optimizer_step_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmuon_adamw.so is not built")


def say(*a):
    """Name the case before a GPU step (flushed, so a failing run still shows it)."""
    print("[case]", *a, file=sys.stderr, flush=True)


def to_np(t: torch.Tensor) -> np.ndarray:
    """Stored values as float32 (bf16 -> fp32 is exact)."""
    return t.detach().float().cpu().numpy()


def f32r(x: float) -> float:
    """A hyperparameter as the library receives it (a C float)."""
    return float(np.float32(x))


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (normal range; 2^-133 floor)."""
    ax = np.abs(x.astype(np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    """Bit equality of float32 arrays, treating every NaN as equal to any NaN."""
    a = np.ascontiguousarray(a, F32)
    b = np.ascontiguousarray(b, F32)
    na, nb = np.isnan(a), np.isnan(b)
    if not np.array_equal(na, nb):
        return False
    return np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))


def first_mismatch(a, b):
    a = np.ascontiguousarray(a, F32).ravel()
    b = np.ascontiguousarray(b, F32).ravel()
    bad = np.nonzero((a.view(np.uint32) != b.view(np.uint32)) & ~(np.isnan(a) & np.isnan(b)))[0]
    if bad.size == 0:
        return None
    i = bad[0]
    return f"{bad.size} mismatches; first at {i}: got {a[i]!r} expected {b[i]!r}"


def weight_excess(w_gpu, w_ora, w_old, c_wd, bf16_storage: bool) -> float:
    """Frobenius norm of the part of |W_gpu - W_oracle| that the update rule
    does not allow without a difference in U.

    Both sides store RNE((mask ? W - c_wd*W : W) - c_lr*U), so
    |W_gpu - W_ora| <= c_lr*|U_gpu - U_ora| + one rounding step of W (+ c_wd*|W|
    where the cautious masks differ). The returned norm must then be at most
    c_lr * ||U_gpu - U_ora||_F <= c_lr * tol * ||U_ora||_F.
    """
    wg = np.asarray(w_gpu, np.float64)
    wo = np.asarray(w_ora, np.float64)
    d = np.abs(wg - wo)
    step = bf16_ulp(np.maximum(np.abs(wg), np.abs(wo))) if bf16_storage else \
        np.spacing(np.maximum(np.abs(wg), np.abs(wo)).astype(np.float32)).astype(np.float64)
    slack = step + abs(float(c_wd)) * np.abs(np.asarray(w_old, np.float64))
    return float(np.linalg.norm(np.maximum(d - slack, 0.0)))
