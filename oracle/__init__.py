"""Oracle for the Muon + AdamW optimizer step: plain, slow, CPU-only.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run anything in this package; the product path
(the HIP library and its Python binding) never does, and this package imports
nothing from it. It is written from the pages' statement of the methods:

* "Chapter 4: The MuonAdamW Optimizer" (autoresearch tutorial): sections
  "The Muon Update Rule", "Polar Express: Newton-Schulz Orthogonalization",
  "The Full Muon Step", "The AdamW Step";
* "3.9 Optimizers: SGD, Adam, Adafactor, Lion, Muon & Shampoo" (llm-stack-book):
  "From Gradient Descent to Momentum", "Implementing AdamW from scratch",
  "Muon: Orthogonalizing the Update";
* "Stuck at the optimizer after figuring out backward()" (nanochat discussion,
  reply by mira687): cautious weight decay, MuonEq, the shape lr multiplier;
* "Muon vs AdamW, Lion and Sophia: a fair race" (mvgpt episode 23), sections
  "Muon" (the scalar view of one polynomial step) and "Lion";
* "3.9 Optimizers", section "Lion: Learning the Sign of the Update" and its
  exercise 5: the Lion step.

Every function is pinned by tests against values the pages print, closed
forms, or library routines (see tests/test_oracle_*.py). No function is
"parity unpinned".
"""
from .bf16 import round_to_bf16, f32_to_bf16_bits, bf16_bits_to_f32  # noqa: F401
from .adamw import adamw_scalars, adamw_step  # noqa: F401
from .lion import lion_scalars, lion_step  # noqa: F401
from .muon import (  # noqa: F401
    KELLER_JORDAN, CLASSICAL_QUINTIC, CUBIC,
    lr_multiplier, momentum_stage, row_sumsq, normalize, newton_schulz,
    post_stage, muon_step, scalar_polynomial, polar_svd, polar_eigh, update_norms,
)
