"""Muon + AdamW optimizer step for AMD Instinct MI355X (gfx950).

The step runs in hand-written HIP kernels behind the C ABI of
``include/muon_adamw.h`` (``libmuon_adamw.so``); this package is its Python
binding. Build the library with ``python -m adamw_optimizer_step_amd.build``.
"""
from .api import (  # noqa: F401
    KELLER_JORDAN, MuonGroup, MuonHParams, adamw_step, bf16_round, lion_step, momentum_stage,
    muon_nonfinite, muon_row_pass, muon_step, muon_step_noalloc, muon_workspace_size, muon_workspace_update,
    newton_schulz, optimizer_step, update_stage,
)
from ._lib import MuonAdamWError, lib  # noqa: F401
from .coefficients import keller_jordan, polar_express  # noqa: F401

# Polar Express table for 5 steps: greedy per-step minimax from singular
# values in [1e-3, 1], each polynomial evaluated at x / 1.01 (headroom for
# bf16 rounding at the top of the spectrum); see ``coefficients``.
POLAR_EXPRESS = tuple(polar_express(5, lower=1e-3, safety=1.01))

__all__ = [
    "KELLER_JORDAN", "POLAR_EXPRESS", "keller_jordan", "polar_express", "MuonGroup", "MuonHParams", "MuonAdamWError", "adamw_step", "lion_step", "muon_step",
    "muon_nonfinite", "muon_row_pass", "muon_step_noalloc", "muon_workspace_size", "muon_workspace_update", "optimizer_step", "lib",
]
