"""Seeded synthetic workloads for the Muon + AdamW optimizer step.

Only random draws and their arrangement into the parameter shapes of each
workload live here. None of the optimizer's arithmetic does: the oracle and the
GPU path both take their inputs from this package and share nothing else.
"""
from .inputs import (  # noqa: F401
    MuonGroupSpec, AdamWSegmentSpec, Workload, WORKLOADS, workload,
    gaussian, kron_spectrum_factors, kron_spectrum_matrix, seed0_gaussian_256x1024,
    rank8_plus_noise_256x1024, materialize, grad_factors,
)
