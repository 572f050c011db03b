"""Muon step for one weight matrix, written out step by step (oracle).

Sources, in the order the step runs:

1. Momentum, sum form ``m <- beta*m + G`` and the Nesterov look-ahead
   ``G + beta*m``: "Chapter 4: The MuonAdamW Optimizer", sections "The Muon
   Update Rule" and "The Full Muon Step"; "3.9 Optimizers ...", section "From
   Gradient Descent to Momentum" (the ``sgd_momentum_step`` listing).
2. Optional MuonEq row equilibration: named as an optional extra of nanochat's
   Muon in "Stuck at the optimizer after figuring out backward()" (reply by
   mira687). Reading used here: each row (output feature) of the look-ahead
   matrix is divided by its Euclidean norm before the Frobenius normalisation.
3. Frobenius normalisation ``X0 = M / (||M||_F + 1e-7)``: "Chapter 4", section
   "Polar Express: Newton-Schulz Orthogonalization"; "3.9 Optimizers", section
   "Muon: Orthogonalizing the Update".
4. ``T`` quintic steps, each the odd polynomial ``a X + b (X X^T) X + c (X
   X^T)^2 X`` with a per-step coefficient triple (same two sections; Polar
   Express uses a different triple at each step, per the nanochat
   discussion), evaluated through the smaller Gram matrix: ``X X^T`` when
   the matrix has no more rows than columns, ``X^T X`` otherwise.
5. Cautious decoupled weight decay and the update ``W - lr_eff*wd*mask*W -
   lr_eff*U`` with ``mask = (U * W >= 0)`` and ``lr_eff = lr *
   sqrt(max(1, rows/cols))``: nanochat discussion (mask and multiplier);
   "Chapter 4", section "The Full Muon Step" (decay uses the weight before
   the update).

Precision modes of the Newton-Schulz part (``precision``):

* ``"f64"``: no rounding anywhere -- the reference for fp32-mode parity;
* ``"f32"``: X0 and every product in binary32 (numpy sgemm);
* ``"bf16"``: the rounding points of the bf16 GPU path. X0 is rounded to
  bf16; the Gram matrix ``A`` (``X X^T``, or ``X^T X`` for a tall matrix) is
  formed exactly (float64 sums of exact products of bf16 values, standing in
  for an fp32 accumulator) and rounded to bf16; ``B = b*A + c*(A A)`` likewise
  from the rounded A, rounded once; ``X' = a*X + B X`` (tall: ``a*X + X B``)
  likewise from the rounded B and X, rounded once.

The elementwise parts (momentum, decay, update) are binary32 with one rounding
per operation and no fused multiply-add; they are the bit-exact contract.
"""
from __future__ import annotations

import math
from typing import Iterable, Sequence, Tuple

import numpy as np

from .bf16 import round_to_bf16

f32 = np.float32
f64 = np.float64

# Coefficient triples printed on the pages.
# Keller Jordan's (a, b, c): "Chapter 4", section "Polar Express: Newton-Schulz
# Orthogonalization"; "3.9 Optimizers", section "Muon: Orthogonalizing the Update".
KELLER_JORDAN = (3.4445, -4.7750, 2.0315)
# Classical quintic Newton-Schulz: "A transformer trained with Muon", section
# "The optimizer, Muon".
CLASSICAL_QUINTIC = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)
# Cubic Newton-Schulz X (3I - X^T X) / 2 written as a quintic with c = 0:
# "Chapter 4", section "Polar Express: Newton-Schulz Orthogonalization".
CUBIC = (1.5, -0.5, 0.0)


def coefficient_schedule(coeffs, ns_steps=None) -> Tuple[Tuple[float, float, float], ...]:
    """Normalise ``coeffs`` to a tuple of per-step triples.

    ``coeffs`` is one triple (repeated ``ns_steps`` times) or a sequence of
    triples (one per step; ``ns_steps`` must then match or be None).
    """
    c = list(coeffs)
    if len(c) == 3 and all(np.isscalar(v) for v in c):
        if ns_steps is None:
            raise ValueError("ns_steps is needed with a single coefficient triple")
        return tuple((float(c[0]), float(c[1]), float(c[2])) for _ in range(int(ns_steps)))
    steps = tuple(tuple(float(v) for v in t) for t in c)
    if ns_steps is not None and len(steps) != int(ns_steps):
        raise ValueError("coefficient table length does not match ns_steps")
    return steps


def lr_multiplier(rows: int, cols: int, scale="sqrt_max1_r_over_c") -> float:
    """Per-matrix lr multiplier.

    * ``"sqrt_max1_r_over_c"`` (or True): ``sqrt(max(1, rows/cols))`` (nanochat
      discussion, reply by mira687);
    * ``"moonshot"``: ``0.2 * sqrt(max(rows, cols))`` ("Muon vs AdamW, Lion and
      Sophia: a fair race", the Muon section);
    * ``"sqrt_max"``: ``sqrt(max(rows, cols))`` ("3.9 Optimizers ...", section
      "Muon: Orthogonalizing the Update");
    * ``"none"`` (or False): 1.
    """
    if scale is True or scale == "sqrt_max1_r_over_c":
        return math.sqrt(max(1.0, rows / cols))
    if scale == "moonshot":
        return 0.2 * math.sqrt(max(rows, cols))
    if scale == "sqrt_max":
        return math.sqrt(max(rows, cols))
    if scale is False or scale == "none":
        return 1.0
    raise ValueError(f"unknown lr scale {scale!r}")


def momentum_stage(g, m, beta: float, nesterov: bool = True):
    """Momentum buffer update and Nesterov look-ahead, binary32.

    Returns ``(m1, mt)`` with ``m1 = beta*m + g`` (the new buffer, before it is
    stored in its own dtype) and ``mt = g + beta*m1`` if ``nesterov`` else
    ``m1``. The look-ahead reads the binary32 ``m1``, not its stored rounding.
    """
    b = f32(beta)
    g = np.asarray(g, dtype=f32)
    m = np.asarray(m, dtype=f32)
    with np.errstate(all="ignore"):
        m1 = b * m + g
        mt = (g + b * m1) if nesterov else m1
    return m1.astype(f32), mt.astype(f32)


def row_sumsq(x) -> np.ndarray:
    """Sum of squares of every row (float64)."""
    x = np.asarray(x, dtype=f64)
    return np.sum(x * x, axis=-1)


def normalize(mt, equilibrate: str = "off", norm_eps: float = 1e-7, eq_eps: float = 1e-7):
    """``X0``: optional row equilibration, then division by the Frobenius norm (float64).

    ``equilibrate == "pre"`` divides row i by ``||row_i|| + eq_eps`` first.
    """
    x = np.asarray(mt, dtype=f64)
    if equilibrate == "pre":
        r = np.sqrt(row_sumsq(x))
        x = x / (r + eq_eps)[:, None]
    fro = math.sqrt(float(np.sum(x * x)))
    return x / (fro + norm_eps)


def _round(x, precision):
    if precision == "f64":
        return np.asarray(x, dtype=f64)
    if precision == "f32":
        return np.asarray(x, dtype=f32)
    if precision == "bf16":
        return round_to_bf16(x).astype(f64)
    raise ValueError(precision)


def newton_schulz(x0, coeffs, precision: str = "f64", ns_steps=None):
    """Quintic Newton-Schulz / Polar Express iteration on ``x0`` (param layout).

    One step replaces X by the odd matrix polynomial
    ``p(X) = a X + b (X X^T) X + c (X X^T)^2 X``: with ``X = U diag(s) V^T`` it
    maps each singular value s to ``a s + b s^3 + c s^5`` and keeps U and V
    ("Muon vs AdamW, Lion and Sophia: a fair race", section "Muon"; "3.9
    Optimizers ...", section "Muon: Orthogonalizing the Update"). Because
    ``(X X^T) X = X (X^T X)``, the polynomial is evaluated through the smaller
    Gram matrix, as both pages prescribe for the cost ("Chapter 4", section
    "Polar Express: Newton-Schulz Orthogonalization"):

    * rows <= cols: ``G = X X^T``, ``B = b G + c G G``, ``p(X) = a X + B X``;
    * rows >  cols: ``G = X^T X``, ``B = b G + c G G``, ``p(X) = a X + X B``.

    Rounding (``precision``): "f64" rounds nowhere; "f32" keeps every array and
    coefficient in binary32 (numpy sgemm); "bf16" rounds ``x0`` to bf16 and
    then, at each step, G, B and the new X once each (exact float64 products of
    bf16 values stand in for the fp32 accumulator; one rounding to binary32,
    then to bf16). The result has ``x0``'s shape.
    """
    steps = coefficient_schedule(coeffs, ns_steps)
    X = _round(x0, precision)
    wide = X.shape[0] <= X.shape[1]
    rnd = (lambda Y: _round(Y, "bf16")) if precision == "bf16" else (lambda Y: Y)
    k = f32 if precision == "f32" else float
    for a, b, c in steps:
        G = rnd(X @ X.T if wide else X.T @ X)
        B = rnd(k(b) * G + k(c) * (G @ G))
        X = rnd(k(a) * X + (B @ X if wide else X @ B))
    return np.ascontiguousarray(X)


def post_stage(w, u, c_lr, c_wd, cautious: bool, decay: bool = True):
    """Cautious decoupled decay and the update, binary32, no fused multiply-add.

    ``mask = (u*w >= 0)`` if ``cautious`` (all ones otherwise; NaN compares
    false, so a NaN product gets no decay). Both terms read the weight before
    the update: ``w1 = mask ? w - c_wd*w : w``, ``w2 = w1 - c_lr*u``.
    ``decay`` False (weight decay 0) skips the decay term entirely.
    Returns ``(w2, mask)``; ``w2`` is binary32, before rounding to the
    parameter's own dtype.
    """
    w = np.asarray(w, dtype=f32)
    u = np.asarray(u, dtype=f32)
    cl, cw = f32(c_lr), f32(c_wd)
    with np.errstate(all="ignore"):
        if cautious:
            mask = (u * w) >= f32(0)
        else:
            mask = np.ones(w.shape, dtype=bool)
        if decay:
            w1 = np.where(mask, w - cw * w, w).astype(f32)
        else:
            w1 = w
        w2 = (w1 - cl * u).astype(f32)
    return w2, mask


def _store(x, dtype: str):
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=f32)
    raise ValueError(dtype)


def muon_step(W, G, M, *, lr: float, momentum: float = 0.95, nesterov: bool = True,
              coeffs=KELLER_JORDAN, ns_steps: int | None = 5, weight_decay: float = 0.0,
              cautious: bool = False, equilibrate: str = "off", precision: str = "bf16",
              param_dtype: str = "bf16", mom_dtype: str = "bf16", norm_eps: float = 1e-7,
              eq_eps: float = 1e-7, lr_scale="sqrt_max1_r_over_c"):
    """One Muon step for one ``rows x cols`` matrix.

    Inputs are arrays holding the stored values (bf16 values as float32).
    Returns a dict with the stored new weight ``W`` and buffer ``M``, the
    update direction ``U`` the decay and update consumed (binary32, param
    layout), ``U_ns`` the Newton-Schulz result before any row scaling after
    the iteration (MuonEq POST, NorMuon), ``X0`` (float64), the mask and the binary32 scalars used.
    """
    W = np.asarray(W, dtype=f32)
    R, C = W.shape
    m1, mt = momentum_stage(G, M, momentum, nesterov)
    M_new = _store(m1, mom_dtype)
    x0 = normalize(mt, "pre" if equilibrate == "pre" else "off", norm_eps, eq_eps)
    U = newton_schulz(x0, coeffs, precision, ns_steps)
    U_ns = np.asarray(U, dtype=f32)
    if equilibrate == "post":
        Uf = np.asarray(U, dtype=f64)
        rho = math.sqrt(float(np.sum(Uf * Uf))) / math.sqrt(R)
        rn = np.sqrt(row_sumsq(Uf))
        U = Uf * (rho / (rn + eq_eps))[:, None]
    elif equilibrate == "rms":
        # NorMuon ("Chapter 4", section "NorMuon: Normalized Muon"): each row
        # divided by its RMS, ||U_i|| / sqrt(cols), plus eq_eps
        Uf = np.asarray(U, dtype=f64)
        rms = np.sqrt(row_sumsq(Uf)) / math.sqrt(C)
        U = Uf / (rms + eq_eps)[:, None]
    u = np.asarray(U, dtype=f32)
    lr_eff = lr * lr_multiplier(R, C, lr_scale)
    c_lr, c_wd = f32(lr_eff), f32(lr_eff * weight_decay)
    w2, mask = post_stage(W, u, c_lr, c_wd, cautious, decay=(weight_decay != 0.0))
    return {"W": _store(w2, param_dtype), "M": M_new, "U": u, "U_ns": U_ns, "X0": x0, "mask": mask,
            "c_lr": c_lr, "c_wd": c_wd, "m1": m1, "mt": mt}


# ----------------------------------------------------------------------------
# exact references used only to pin the iteration
# ----------------------------------------------------------------------------

def scalar_polynomial(s, coeffs, ns_steps=None):
    """The composed scalar map ``s <- a s + b s^3 + c s^5`` over the schedule.

    One Newton-Schulz step acts on each singular value by this odd quintic
    ("Muon vs AdamW, Lion and Sophia: a fair race", section "Muon";
    "Chapter 4", section "Why 5 Steps?").
    """
    s = np.asarray(s, dtype=f64)
    for a, b, c in coefficient_schedule(coeffs, ns_steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def update_norms(w_old, w_new):
    """``(||w_new - w_old||_F, ||w_old||_F)`` in float64: the size of one step
    and of the weight it was taken from, whose ratio is the per-layer
    diagnostic of "3.9 Optimizers ...", section "Large-batch training: LARS,
    LAMB and the trust ratio". Both arrays hold the stored values (w_new
    after rounding to the parameter's type)."""
    a = np.asarray(w_old, dtype=f64)
    b = np.asarray(w_new, dtype=f64)
    d = b - a
    return math.sqrt(float(np.sum(d * d))), math.sqrt(float(np.sum(a * a)))


def polar_svd(M):
    """Exact polar factor ``U V^T`` from the thin SVD (singular values set to 1).

    "Chapter 4", section "The Muon Update Rule"; "3.9 Optimizers", section
    "Muon: Orthogonalizing the Update".
    """
    U, _, Vt = np.linalg.svd(np.asarray(M, dtype=f64), full_matrices=False)
    return U @ Vt


def polar_eigh(M):
    """``(M M^T)^{-1/2} M`` via a symmetric eigendecomposition.

    "3.9 Optimizers", section "Muon: Orthogonalizing the Update" and exercise 6(b).
    Needs full row rank; a matrix with more rows than columns is handled through
    its transpose.
    """
    M = np.asarray(M, dtype=f64)
    if M.shape[0] > M.shape[1]:
        return polar_eigh(M.T).T
    lam, Q = np.linalg.eigh(M @ M.T)
    return (Q * (1.0 / np.sqrt(lam))) @ Q.T @ M
