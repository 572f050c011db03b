"""The largest single-GPU share at full size: 32 layers of d=4096 matrices,
128 x 4096^2, 32 x 16384x4096 (tall) and 32 x 4096x16384, bf16, in one
Muon call launched as the benchmark launches its workloads.

An oracle run of a 4096 x 16384 matrix takes minutes on the host, so this
size is checked through properties that hold at any size:

* the gradients are U diag(s) V^T with U, V Kronecker products of small
  orthogonal factors, so with zero momentum and no row scaling the iteration's
  exact result is U phi(s/||s||) V^T, phi the composed quintic (the scalar
  form of the iteration, "Muon vs AdamW, Lion and Sophia: a fair race",
  section "Muon"). Rotating the GPU result by U^T . V costs O(mn(p+q)) with
  the factors, and the rotated matrix must be diag(phi) up to bf16 rounding;
* with the workload's own settings (cautious decay, MuonEq before the
  iteration, random momentum): the stored momentum is bit-exact on sampled
  rows, everything is finite and the update's spectral norm stays inside the
  polynomial's band.

Tolerance of the closed-form check: the stored bf16 gradient carries a
relative rounding of about 2^-9, which the iteration amplifies in the small
singular directions, and every bf16 rounding point inside the iteration adds
to it. The bf16-emulating oracle itself lands 0.002 (one step) to 0.044
(five steps) from the closed form on these matrices
(tests/golden/closed_form_bf16_error.json, written by the script beside it
from the oracle alone); the GPU result may be at most 1.02 times the
oracle's distance for the same matrix. The 64 largest directions are checked
to the bf16 bar of 2e-2.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import bits_equal, f32r, first_mismatch, need_gpu, say, to_np
from workloads import grad_factors, materialize, workload

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
KJ = (3.4445, -4.7750, 2.0315)


# the GPU's distance to the closed form may exceed the bf16 oracle's own by this
# factor: measured on MI355X, the two agree to 3-4 significant digits at
# ns_steps 1, 3 and 5 (the largest GPU/oracle ratio over the 18 matrices was
# 1.0015), so 2% is the slack kept for rounding differences
RATIO = 1.02
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_form_bf16_error.json")


def _oracle_distance():
    """(ns_steps, group, matrix) -> the oracle's relative distance to the closed form."""
    with open(GOLDEN) as fh:
        return {(c.get("ns_steps", 5), c["group"], c["matrix"]): c["rel_fro"] for c in json.load(fh)["cases"]}


def _hp(M, wl, **kw):
    d = dict(lr=f32r(wl.lr), momentum=f32r(wl.momentum), weight_decay=f32r(wl.weight_decay),
             nesterov=wl.nesterov, ns_steps=wl.ns_steps, coeffs=KJ, cautious=wl.cautious,
             equilibrate=wl.equilibrate, ns_precision=wl.ns_precision, norm_eps=f32r(1e-7), eq_eps=f32r(1e-7))
    d.update(kw)
    return M.MuonHParams(**d)


def _rotate(Y, factors):
    """U^T Y V for U = kron(U1, U2), V = kron(V1, V2), float64 on the GPU."""
    U1, U2, V1, V2, _ = (t.to(DEV, torch.float64).contiguous() for t in factors)
    r1, m1 = U1.shape
    r2, m2 = U2.shape
    c1, c2 = V1.shape[0], V2.shape[0]
    T = Y.to(torch.float64).reshape(r1, r2, c1, c2)
    T = torch.einsum("ia,ijkl->ajkl", U1, T).contiguous()
    T = torch.einsum("jb,ajkl->abkl", U2, T).contiguous()
    T = torch.einsum("kc,abkl->abcl", V1, T).contiguous()
    T = torch.einsum("ld,abcl->abcd", V2, T).contiguous()
    return T.reshape(m1 * m2, m1 * m2)


@pytest.mark.parametrize("ns_steps", [1, 3, 5])
def test_largest_share_closed_form(ns_steps):
    """The ns_steps sweep {1, 3, 5} of the nanochat discussion ("Stuck at the
    optimizer after figuring out backward()", reply by mira687) at the
    largest single-GPU share."""
    need_gpu()
    import adamw_optimizer_step_amd as M
    wl = workload("c5_32L_d4096").scaled(mom_init="zero", equilibrate="off", ns_steps=ns_steps)
    say("largest share: inputs", ns_steps)
    data = materialize(wl, device=DEV, seed=0)
    mgs = [M.MuonGroup(d["W"], d["G"], d["M"]) for d in data["muon"]]
    hp = _hp(M, wl)
    ref = _oracle_distance()
    say("largest share: step", ns_steps, [m.count for m in mgs])
    ws = M.muon_step(mgs, hp)
    torch.cuda.synchronize()
    for gi, d in enumerate(data["muon"]):
        assert torch.isfinite(d["W"]).all(), f"group {gi}: non-finite weights"
        for k in sorted({0, d["W"].shape[0] - 1}):
            f = grad_factors(wl, gi, k, seed=0)
            s = f[4].numpy()
            phi = torch.from_numpy(O.scalar_polynomial(s / np.linalg.norm(s), KJ, wl.ns_steps)).to(DEV)
            Y = M.muon_workspace_update(mgs, hp, ws, gi, k)
            say("largest share: closed form", gi, k, tuple(Y.shape))
            D = _rotate(Y, f)
            err = float(torch.linalg.matrix_norm(D - torch.diag(phi)) / torch.linalg.vector_norm(phi))
            bound = RATIO * ref[(ns_steps, gi, k)]
            say("largest share: closed form", ns_steps, gi, k, f"gpu {err:.5f}", f"oracle {ref[(ns_steps, gi, k)]:.5f}")
            assert err <= bound, f"group {gi} matrix {k}: relative distance to U phi V^T {err:.4f} > {bound:.4f}"
            top = float((torch.diagonal(D)[:64] - phi[:64]).abs().div(phi[:64]).max())
            assert top <= 2e-2, f"group {gi} matrix {k}: top-64 singular values off by {top:.4f}"
    del data, mgs, ws
    torch.cuda.empty_cache()


def _spectral_norm(X, iters=30):
    X = X.to(torch.float32)
    v = torch.randn(X.shape[1], device=DEV, generator=torch.Generator(device=DEV).manual_seed(1))
    for _ in range(iters):
        v = X.t().mv(X.mv(v))
        v = v / torch.linalg.vector_norm(v)
    return float(torch.linalg.vector_norm(X.mv(v)))


def test_largest_share_configured_step():
    need_gpu()
    import adamw_optimizer_step_amd as M
    wl = workload("c5_32L_d4096")
    say("largest share (configured): inputs")
    data = materialize(wl, device=DEV, seed=1)
    rows_idx = {}
    before = []
    for gi, d in enumerate(data["muon"]):
        n, R, _ = d["W"].shape
        ks = sorted({0, n - 1})
        rs = sorted({0, R // 2, R - 1})
        rows_idx[gi] = (ks, rs)
        before.append([(to_np(d["G"][k, rs]), to_np(d["M"][k, rs])) for k in ks])
    mgs = [M.MuonGroup(d["W"], d["G"], d["M"]) for d in data["muon"]]
    hp = _hp(M, wl)
    say("largest share (configured): step", [m.count for m in mgs])
    ws = M.muon_step(mgs, hp)
    torch.cuda.synchronize()
    band = float(O.scalar_polynomial(np.linspace(1e-4, 1.0, 100001), KJ, wl.ns_steps).max())
    for gi, d in enumerate(data["muon"]):
        assert torch.isfinite(d["W"]).all() and torch.isfinite(d["M"].float()).all(), f"group {gi}"
        ks, rs = rows_idx[gi]
        for k, (g, m) in zip(ks, before[gi]):
            m1, _ = O.momentum_stage(g, m, hp.momentum, hp.nesterov)
            got = to_np(d["M"][k, rs])
            assert bits_equal(got, O.round_to_bf16(m1)), first_mismatch(got, O.round_to_bf16(m1))
            U = M.muon_workspace_update(mgs, hp, ws, gi, k)
            say("largest share (configured): spectral norm", gi, k)
            # the polynomial maps (0, 1] into (0, band]; bf16 rounding adds a little
            assert _spectral_norm(U) <= band * 1.03, f"group {gi} matrix {k}"
    del data, mgs, ws
    torch.cuda.empty_cache()
