"""Writes closed_form_bf16_error.json: how far the bf16-emulating oracle lands
from the exact result U phi(s/||s||) V^T on the largest single-GPU share
(32 layers of d=4096: groups of 4096^2, 16384x4096 and 4096x16384 matrices
with power-law spectrum s_i ~ 1/i), for the matrices the full-size GPU test
checks (first and last of every group, input seed 0, zero momentum, no row
equilibration, 1, 3 and 5 steps of the (3.4445, -4.7750, 2.0315) quintic:
the ns_steps sweep of the nanochat discussion "Stuck at the optimizer after
figuring out backward()", reply by mira687).

The exact result follows from the scalar form of the iteration: every step
maps each singular value through the same odd quintic and leaves the
singular vectors alone ("Muon vs AdamW, Lion and Sophia: a fair race",
section "Muon"). The distance is the relative Frobenius norm of
U^T Y V - diag(phi), computed with the Kronecker factors.

Run from the repository root: python tests/golden/make_closed_form_bf16_error.py
(about twenty minutes on eight host cores). Calls only the oracle and the
seeded input generators.
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from workloads import grad_factors, kron_spectrum_matrix, workload  # noqa: E402

import torch  # noqa: E402

KJ = (3.4445, -4.7750, 2.0315)
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "closed_form_bf16_error.json")


def rotate(Y, factors):
    """U^T Y V with U = kron(U1, U2), V = kron(V1, V2), mode by mode."""
    U1, U2, V1, V2, _ = (t.numpy() for t in factors)
    r1, m1 = U1.shape
    r2, m2 = U2.shape
    c1, c2 = V1.shape[0], V2.shape[0]
    T = Y.reshape(r1, r2, c1, c2)
    T = np.einsum("ia,ijkl->ajkl", U1, T, optimize=True)
    T = np.einsum("jb,ajkl->abkl", U2, T, optimize=True)
    T = np.einsum("kc,abkl->abcl", V1, T, optimize=True)
    T = np.einsum("ld,abcl->abcd", V2, T, optimize=True)
    return T.reshape(m1 * m2, m1 * m2)


def main():
    wl = workload("c5_32L_d4096")
    cases = []
    for gi, spec in enumerate(wl.muon_groups):
        for k in sorted({0, spec.count - 1}):
            f = grad_factors(wl, gi, k, seed=0)
            g = O.round_to_bf16(kron_spectrum_matrix(f, "cpu", torch.float64).numpy().astype(np.float32))
            _, mt = O.momentum_stage(g, np.zeros_like(g), wl.momentum, wl.nesterov)
            x0 = O.normalize(mt, "off", 1e-7)
            s = f[4].numpy()
            for T in (1, 3, 5):
                t0 = time.time()
                Y = O.newton_schulz(x0, KJ, "bf16", T).astype(np.float64)
                D = rotate(Y, f)
                phi = O.scalar_polynomial(s / np.linalg.norm(s), KJ, T)
                err = float(np.linalg.norm(D - np.diag(phi)) / np.linalg.norm(phi))
                top = float(np.max(np.abs(np.diag(D)[:64] - phi[:64]) / phi[:64]))
                cases.append({"ns_steps": T, "group": gi, "rows": spec.rows, "cols": spec.cols, "matrix": k,
                              "rel_fro": round(err, 6), "top64_rel": round(top, 6)})
                print(cases[-1], f"{time.time() - t0:.0f}s", flush=True)
    doc = {
        "source": "scalar form of the quintic iteration: singular values pass through the composed "
                  "polynomial, singular vectors are kept -- Muon vs AdamW, Lion and Sophia: a fair race, "
                  "section 'Muon'",
        "what": "relative Frobenius distance of the bf16-emulating oracle's Newton-Schulz output from "
                "U phi(s/||s||) V^T, and the largest relative error among the 64 largest singular values",
        "workload": "32 layers d=4096, input seed 0, zero momentum, equilibration off, 1, 3 and 5 steps of "
                    "(3.4445, -4.7750, 2.0315)",
        "command": "python tests/golden/make_closed_form_bf16_error.py",
        "cases": cases,
    }
    with open(OUT, "w") as fh:
        json.dump(doc, fh, indent=1)
        fh.write("\n")


if __name__ == "__main__":
    main()
