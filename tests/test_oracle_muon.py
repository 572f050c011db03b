"""Pins for the oracle's Muon step (CPU only).

The iteration is tied to things other than itself:

* the exact polar factor U V^T by SVD and by (M M^T)^{-1/2} M (two routes that
  pin each other), which the classical quintic and the cubic converge to;
* the closed form of the iteration: for G = U diag(s) V^T the result is
  U diag(phi(s / ||s||)) V^T with phi the composed scalar quintic, for wide and
  tall shapes and for a schedule whose steps differ (the order matters);
* the page tests and figures: the QR-built spectrum test of the mvgpt episode
  ("Muon vs AdamW, Lion and Sophia: a fair race", section "Muon"), the 5x8
  spread of the viv-lang notebook ("A transformer trained with Muon", section
  "The optimizer, Muon"), the condition numbers and cosines of the nanochat
  discussion, the lr multiplier (x2 for c_fc, x1 for c_proj);
* hand-worked momentum and cautious-decay cases (tests/golden);
* torch.optim.Muon on CPU as an independent implementation.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from workloads import (kron_spectrum_factors, kron_spectrum_matrix, rank8_plus_noise_256x1024,
                       seed0_gaussian_256x1024)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _cond(x):
    s = np.linalg.svd(np.asarray(x, np.float64), compute_uv=False)
    return s[0] / s[-1]


def _cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def _rel(a, b):
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


def _spectrum_matrix(rows, cols, s, seed):
    rng = np.random.default_rng(seed)
    m = min(rows, cols)
    U, _ = np.linalg.qr(rng.standard_normal((rows, m)))
    V, _ = np.linalg.qr(rng.standard_normal((cols, m)))
    return U, V, (U * s) @ V.T


# ------------------------------------------------------------ exact polar factor

@pytest.mark.parametrize("shape", [(2, 3), (8, 5), (16, 16), (64, 256), (96, 40)])
def test_polar_routes_agree(shape):
    rng = np.random.default_rng(sum(shape))
    M = rng.standard_normal(shape)
    P1, P2 = O.polar_svd(M), O.polar_eigh(M)
    assert _rel(P2, P1) < 1e-10
    m = min(shape)
    gram = P1 @ P1.T if shape[0] <= shape[1] else P1.T @ P1
    assert np.allclose(gram, np.eye(m), atol=1e-12)


@pytest.mark.parametrize("shape", [(2, 3), (8, 5), (24, 24), (64, 256), (200, 48)])
@pytest.mark.parametrize("coeffs,steps", [(O.CLASSICAL_QUINTIC, 40), (O.CUBIC, 60)])
def test_classical_iterations_converge_to_polar(shape, coeffs, steps):
    """Classical quintic and cubic Newton-Schulz reach U V^T (cond <= 100)."""
    m = min(shape)
    s = np.geomspace(1.0, 1e-2, m)
    _, _, M = _spectrum_matrix(shape[0], shape[1], s, 11 * m)
    X = O.newton_schulz(O.normalize(M), coeffs, "f64", steps)
    assert _rel(X, O.polar_svd(M)) < 1e-12


# ------------------------------------------------------------ closed form

@pytest.mark.parametrize("shape", [(16, 64), (64, 16), (48, 48), (1, 9), (9, 1)])
def test_iteration_closed_form_keller_jordan(shape):
    m = min(shape)
    s = np.geomspace(3.0, 0.02, m)
    U, V, M = _spectrum_matrix(shape[0], shape[1], s, 3 + m)
    X = O.newton_schulz(O.normalize(M), O.KELLER_JORDAN, "f64", 5)
    sn = s / (np.linalg.norm(s) + 1e-7)
    expect = (U * O.scalar_polynomial(sn, O.KELLER_JORDAN, 5)) @ V.T
    assert _rel(X, expect) < 1e-12
    # the iteration keeps the singular vectors: U^T X V is diagonal
    D = U.T @ X @ V
    assert np.max(np.abs(D - np.diag(np.diag(D)))) < 1e-12


def test_iteration_closed_form_per_step_schedule_order():
    """A schedule of different triples composes in order; reversing it differs."""
    sched = [O.KELLER_JORDAN, (2.0, -1.5, 0.5), O.CUBIC, (3.0, -3.2, 1.2), O.CLASSICAL_QUINTIC]
    s = np.geomspace(1.0, 0.05, 32)
    U, V, M = _spectrum_matrix(32, 96, s, 99)
    X = O.newton_schulz(O.normalize(M), sched, "f64")
    sn = s / (np.linalg.norm(s) + 1e-7)
    assert _rel(X, (U * O.scalar_polynomial(sn, sched)) @ V.T) < 1e-12
    rev = (U * O.scalar_polynomial(sn, sched[::-1])) @ V.T
    assert _rel(X, rev) > 1e-3


def test_kron_spectrum_workload_closed_form():
    """The Kronecker-structured workload gradients obey the closed form too."""
    f = kron_spectrum_factors(64, 256, "spectrum_inv", 1e-3, seed=4)
    G = kron_spectrum_matrix(f, dtype=torch.float64).numpy()
    U = np.kron(f[0].numpy(), f[1].numpy())
    V = np.kron(f[2].numpy(), f[3].numpy())
    s = f[4].numpy()
    assert abs(np.sqrt(np.mean(G * G)) - 1e-3) < 1e-9
    X = O.newton_schulz(O.normalize(G), O.KELLER_JORDAN, "f64", 5)
    sn = s / (np.linalg.norm(s) + 1e-7)
    assert _rel(X, (U * O.scalar_polynomial(sn, O.KELLER_JORDAN, 5)) @ V.T) < 1e-10


# ------------------------------------------------------------ page tests and figures

def test_mvgpt_spectrum_test_diagonal_band():
    """QR-built U, V with singular values from 0.1 to 10: result diagonal in U, V
    with diagonal entries between 0.6 and 1.2 (mvgpt episode, section "Muon")."""
    s = np.geomspace(10.0, 0.1, 32)
    U, V, M = _spectrum_matrix(32, 64, s, 2024)
    X = O.newton_schulz(O.normalize(M), O.KELLER_JORDAN, "f64", 5)
    D = U.T @ X @ V
    off = D - np.diag(np.diag(D))
    assert np.max(np.abs(off)) < 1e-10
    assert 0.6 <= np.diag(D).min() and np.diag(D).max() <= 1.2


def test_viv_notebook_5x8_spread(golden_dir):
    ref = json.load(open(os.path.join(golden_dir, "viv_notebook_spread.json")))
    s = np.geomspace(ref["sigma_max"], ref["sigma_min"], 5)
    U, V, M = _spectrum_matrix(5, 8, s, 8)
    out = {}
    for name, co in (("keller_jordan", O.KELLER_JORDAN), ("classical", O.CLASSICAL_QUINTIC)):
        X = O.newton_schulz(O.normalize(M), co, "f64", 5)
        sv = np.linalg.svd(X, compute_uv=False)
        out[name] = (sv.min(), sv.max(), sv.max() / sv.min())
    kmin, kmax, kspread = out["keller_jordan"]
    cmin, cmax, cspread = out["classical"]
    kj = ref["keller_jordan"]
    assert abs(kspread - kj["spread"]) < 0.25 * kj["spread"]
    assert abs(kmin - kj["min"]) < 0.05 and abs(kmax - kj["max"]) < 0.1
    assert abs(cspread - ref["classical"]["spread"]) < 0.1 * ref["classical"]["spread"]
    assert cmax <= 1.0 + 1e-12          # the classical map stays below 1
    assert kspread < cspread / 10


def test_nanochat_iid_figures(golden_dir):
    ref = json.load(open(os.path.join(golden_dir, "nanochat_discussion_measurements.json")))
    fig = ref["iid_seed0_256x1024"]
    G = seed0_gaussian_256x1024().numpy()
    assert round(_cond(G), 2) == fig["cond_G"]
    X = O.newton_schulz(O.normalize(G), O.KELLER_JORDAN, "f64", 5)
    P = O.polar_svd(G)
    # the page's Polar Express result lies between five Keller-Jordan steps and
    # the exact polar factor, in both figures
    assert _cos(G, X) < fig["cos_G_update"] < _cos(G, P)
    assert 1.0 < fig["cond_update"] < _cond(X)


def test_nanochat_condition_collapse_with_ns_steps(golden_dir):
    ref = json.load(open(os.path.join(golden_dir, "nanochat_discussion_measurements.json")))
    sweep = ref["ns_steps_sweep"]
    G = rank8_plus_noise_256x1024().numpy()
    assert 500 < _cond(G) < 1000                       # page: 721 for its own draw
    x0 = O.normalize(G)
    conds = {T: _cond(O.newton_schulz(x0, O.KELLER_JORDAN, "f64", T)) for T in (1, 3, 5)}
    assert conds[1] > conds[3] > conds[5]
    assert abs(conds[1] - sweep["cond_T1"]) < 0.05 * sweep["cond_T1"]  # one step barely moves it
    assert conds[5] < 5.0
    U5 = O.newton_schulz(x0, O.KELLER_JORDAN, "f64", 5)
    c1 = _cos(O.newton_schulz(x0, O.KELLER_JORDAN, "f64", 1), U5)
    c3 = _cos(O.newton_schulz(x0, O.KELLER_JORDAN, "f64", 3), U5)
    assert c1 < c3 < 1.0


def test_nanochat_muoneq_reading(golden_dir):
    """Removing row equilibration moves the direction by cos 0.986 on the page.
    Row equilibration before the iteration (the reading taken) moves it by that
    order on the two page inputs; a row rescale after it cannot (cos > 0.999)."""
    ref = json.load(open(os.path.join(golden_dir, "nanochat_discussion_measurements.json")))
    target = ref["muoneq_removed_cos"]
    pre, post = [], []
    for G in (seed0_gaussian_256x1024().numpy(), rank8_plus_noise_256x1024().numpy()):
        U0 = O.newton_schulz(O.normalize(G), O.KELLER_JORDAN, "f64", 5)
        Up = O.newton_schulz(O.normalize(G, "pre"), O.KELLER_JORDAN, "f64", 5)
        pre.append(_cos(U0, Up))
        rho = np.linalg.norm(U0) / math.sqrt(U0.shape[0])
        Uq = U0 * (rho / (np.linalg.norm(U0, axis=1) + 1e-7))[:, None]
        post.append(_cos(U0, Uq))
    assert min(pre) < target < max(pre)
    assert min(post) > 0.999 > target


def test_lr_multiplier_page_values(golden_dir):
    ref = json.load(open(os.path.join(golden_dir, "nanochat_discussion_measurements.json")))
    assert O.lr_multiplier(4096, 1024) == ref["lr_multiplier"]["c_fc_4d_x_d"]
    assert O.lr_multiplier(1024, 4096) == ref["lr_multiplier"]["c_proj_d_x_4d"]
    assert O.lr_multiplier(1024, 1024) == 1.0


# ------------------------------------------------------------ invariances, edge cases

def test_scale_invariance_and_zero_gradient():
    G = seed0_gaussian_256x1024().numpy()[:64, :128].astype(np.float64)
    X = O.newton_schulz(O.normalize(G), O.KELLER_JORDAN, "f64", 5)
    for a in (1e-3, 7.5, 1e4):
        assert _rel(O.newton_schulz(O.normalize(a * G), O.KELLER_JORDAN, "f64", 5), X) < 1e-5
    Z = np.zeros((8, 16))
    assert not np.any(O.normalize(Z))
    r = O.muon_step(np.ones((8, 16), np.float32), Z, Z, lr=0.1, weight_decay=0.5,
                    precision="bf16", param_dtype="f32", mom_dtype="f32")
    assert np.all(np.isfinite(r["W"])) and not np.any(r["U"])
    assert np.all(r["W"] == np.float32(1) - np.float32(0.1 * 0.5) * np.float32(1))


def test_sum_and_ema_momentum_same_first_direction():
    """From zeroed state the sum form (1+b)G and the EMA form (1-b^2)G point the
    same way, so their updates agree (normalisation removes the scale)."""
    G = rank8_plus_noise_256x1024().numpy()[:96]
    m1, mt = O.momentum_stage(G, np.zeros_like(G), 0.95, True)
    a = O.newton_schulz(O.normalize(mt), O.KELLER_JORDAN, "f64", 5)
    b = O.newton_schulz(O.normalize((1 - 0.95 ** 2) * G.astype(np.float64)), O.KELLER_JORDAN,
                        "f64", 5)
    assert _rel(a, b) < 1e-5


def test_ns_steps_zero_returns_x0():
    G = seed0_gaussian_256x1024().numpy()[:32, :48]
    x0 = O.normalize(G)
    assert np.array_equal(O.newton_schulz(x0, O.KELLER_JORDAN, "f64", 0), x0)
    assert abs(np.linalg.norm(x0) - 1.0) < 1e-6


def test_equilibrate_pre_rows_equal_norm():
    G = rank8_plus_noise_256x1024().numpy()[:64]
    x0 = O.normalize(G, "pre")
    rn = np.linalg.norm(x0, axis=1)
    assert np.allclose(rn, 1.0 / math.sqrt(64), rtol=1e-6)


def test_precision_modes_ordering():
    """fp32 sits within 1e-5 of fp64; bf16 rounding points land near 1e-2."""
    G = seed0_gaussian_256x1024().numpy()
    x0 = O.normalize(G)
    u64 = O.newton_schulz(x0, O.KELLER_JORDAN, "f64", 5)
    assert _rel(O.newton_schulz(x0, O.KELLER_JORDAN, "f32", 5), u64) < 1e-5
    e16 = _rel(O.newton_schulz(x0, O.KELLER_JORDAN, "bf16", 5), u64)
    assert 1e-3 < e16 < 3e-2


# ------------------------------------------------------------ hand-worked elementwise cases

def _num(v):
    return {"nan": np.nan, "inf": np.inf, "-inf": -np.inf}.get(v, v) if isinstance(v, str) else v


def test_momentum_hand_cases(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "momentum_cases.json")))["cases"]
    for c in cases:
        m1, mt = O.momentum_stage(np.float32([c["g"]]), np.float32([c["m"]]), c["beta"],
                                  c["nesterov"])
        assert m1[0] == c["m1"] and mt[0] == c["mt"], c


def test_post_stage_hand_cases(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "post_stage_cases.json")))["cases"]
    for c in cases:
        w2, mask = O.post_stage(np.float32([_num(c["w"])]), np.float32([_num(c["u"])]),
                                c["c_lr"], c["c_wd"], c["cautious"])
        assert bool(mask[0]) == c["mask"], c
        e = _num(c["w2"])
        if isinstance(e, float) and math.isnan(e):
            assert math.isnan(w2[0]), c
        else:
            assert w2[0] == e, c


def test_post_stage_signed_zero_and_subnormal_mask():
    tiny = np.float32(1e-45)
    w = np.float32([0.0, -0.0, tiny, -tiny, 1.0])
    u = np.float32([-1.0, 1.0, tiny, tiny, -0.0])
    _, mask = O.post_stage(w, u, 0.5, 0.25, True)
    # 0*(-1) = -0 >= 0; -0*1 = -0 >= 0; tiny*tiny underflows to +0; -tiny*tiny -> -0; 1*-0 = -0
    assert mask.tolist() == [True, True, True, True, True]


# ------------------------------------------------------------ full step vs torch.optim.Muon

@pytest.mark.parametrize("shape", [(64, 64), (256, 64), (64, 256)])
def test_full_step_matches_torch_muon(shape):
    """cos >= 0.99 and norm within 5% against torch.optim.Muon (bf16 iteration),
    one step from zero momentum, weight decay 0 (mvgpt episode, section "Muon")."""
    gen = torch.Generator().manual_seed(shape[0] * 7 + shape[1])
    W0 = torch.randn(*shape, generator=gen) * 0.02
    G = torch.randn(*shape, generator=gen) * 1e-3
    p = torch.nn.Parameter(W0.clone())
    opt = torch.optim.Muon([p], lr=0.02, weight_decay=0.0, momentum=0.95, nesterov=True,
                           ns_coefficients=O.KELLER_JORDAN, eps=1e-7, ns_steps=5)
    p.grad = G.clone()
    opt.step()
    d_torch = (p.detach() - W0).numpy().astype(np.float64)
    r = O.muon_step(W0.numpy(), G.numpy(), np.zeros(shape, np.float32), lr=0.02,
                    momentum=0.95, nesterov=True, coeffs=O.KELLER_JORDAN, ns_steps=5,
                    precision="f64", param_dtype="f32", mom_dtype="f32")
    d_ours = r["W"].astype(np.float64) - W0.numpy().astype(np.float64)
    assert _cos(d_ours, d_torch) >= 0.99
    assert abs(np.linalg.norm(d_ours) / np.linalg.norm(d_torch) - 1) <= 0.05


def test_full_step_bookkeeping_bf16():
    """Stored buffer = RNE(m1), weight = RNE(post(W, U)), scalars from fp64."""
    gen = torch.Generator().manual_seed(3)
    W = torch.randn(96, 32, generator=gen).to(torch.bfloat16).float().numpy()
    G = (torch.randn(96, 32, generator=gen) * 1e-3).to(torch.bfloat16).float().numpy()
    M = (torch.randn(96, 32, generator=gen) * 3e-3).to(torch.bfloat16).float().numpy()
    r = O.muon_step(W, G, M, lr=0.02, weight_decay=0.01, cautious=True, equilibrate="pre",
                    precision="bf16")
    assert r["c_lr"] == np.float32(0.02 * math.sqrt(3.0))
    assert r["c_wd"] == np.float32(0.02 * math.sqrt(3.0) * 0.01)
    assert np.array_equal(r["M"], O.round_to_bf16(r["m1"]))
    w2, _ = O.post_stage(W, r["U"], r["c_lr"], r["c_wd"], True)
    assert np.array_equal(r["W"], O.round_to_bf16(w2))
    assert np.array_equal(O.round_to_bf16(r["U"]), r["U"])   # bf16 mode: U holds bf16 values


# ---------------------------------------------------------------- scale variants

def test_lr_multiplier_values():
    # nanochat: x2 for the 4096 x 1024 c_fc, x1 for the 1024 x 4096 c_proj;
    # Moonshot 0.2 sqrt(max side); sqrt(max side)
    assert O.lr_multiplier(4096, 1024) == 2.0 and O.lr_multiplier(1024, 4096) == 1.0
    assert O.lr_multiplier(4096, 1024, "moonshot") == pytest.approx(0.2 * 64)
    assert O.lr_multiplier(1024, 4096, "sqrt_max") == 64.0
    assert O.lr_multiplier(7, 3, "none") == 1.0 and O.lr_multiplier(7, 3, False) == 1.0
    with pytest.raises(ValueError):
        O.lr_multiplier(2, 2, "bogus")


@pytest.mark.parametrize("shape", [(48, 160), (160, 48)])
@pytest.mark.parametrize("scale,rms", [("moonshot", 0.2), ("sqrt_max", 1.0)])
def test_scaled_step_rms_of_an_orthogonal_update(shape, scale, rms):
    # A semi-orthogonal R x C update has Frobenius norm sqrt(min(R, C)), so its
    # entries' RMS is 1/sqrt(max(R, C)): with Moonshot's 0.2 sqrt(max side) the
    # step's RMS is 0.2 lr ("Muon vs AdamW, Lion and Sophia: a fair race"),
    # with sqrt(max side) it is lr ("3.9 Optimizers ...").
    R, C = shape
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((R, C)) * 0.02).astype(np.float32)
    G = rng.standard_normal((R, C)).astype(np.float32)
    Z = np.zeros_like(W)
    r = O.muon_step(W, G, Z, lr=0.01, coeffs=O.CLASSICAL_QUINTIC, ns_steps=30, precision="f64",
                    param_dtype="f32", mom_dtype="f32", lr_scale=scale)
    d = (W.astype(np.float64) - r["W"].astype(np.float64)) / 0.01
    assert math.sqrt(float(np.mean(d * d))) == pytest.approx(rms, rel=2e-3)


def test_normuon_rows_have_rms_lr():
    # NorMuon ("Chapter 4", section "NorMuon: Normalized Muon"): every row of
    # the step has RMS lr whatever the spectrum (eps 1e-8 aside)
    rng = np.random.default_rng(6)
    R, C = 40, 120
    W = np.zeros((R, C), np.float32)
    G = (rng.standard_normal((R, 8)) @ rng.standard_normal((8, C))).astype(np.float32)
    Z = np.zeros_like(W)
    r = O.muon_step(W, G, Z, lr=0.01, equilibrate="rms", eq_eps=1e-8, precision="f64", param_dtype="f32",
                    mom_dtype="f32", lr_scale="none")
    d = -r["W"].astype(np.float64) / 0.01
    row_rms = np.sqrt(np.mean(d * d, axis=1))
    assert np.allclose(row_rms, 1.0, rtol=1e-5)
    # the row scaling follows the iteration: U_ns is the plain result
    assert not np.allclose(np.sqrt(np.mean(r["U_ns"].astype(np.float64) ** 2, axis=1)), 1.0, rtol=1e-2)


def test_update_norms_hand_case():
    # step [[0, 1], [2, 0]] from a weight of norm 5 (3-4-5): sizes sqrt(5) and 5
    d, w = O.update_norms([[3.0, 0.0], [0.0, 4.0]], [[3.0, 1.0], [2.0, 4.0]])
    assert d == math.sqrt(5.0) and w == 5.0


def test_update_norms_pure_decay_ratio_is_the_decay():
    # w_new = (1 - c) w with c = 2^-7 and dyadic w: every product is exact, so
    # the ratio ||delta|| / ||w|| is exactly c
    rng = np.random.default_rng(4)
    w = (rng.integers(-512, 513, (64, 96)) / 256.0).astype(np.float32)
    c = 2.0 ** -7
    d, n = O.update_norms(w, (w * np.float32(1.0 - c)).astype(np.float32))
    assert abs(d / n - c) <= 1e-15


def test_update_norms_orthogonal_step():
    # a step on entries where the weight is zero: ||w_new||^2 = ||w||^2 + ||delta||^2
    rng = np.random.default_rng(5)
    w = rng.standard_normal((32, 32))
    w[:, 16:] = 0.0
    step = np.zeros_like(w)
    step[:, 16:] = rng.standard_normal((32, 16))
    d, n = O.update_norms(w, w + step)
    n_new, _ = O.update_norms(np.zeros_like(w), w + step)
    assert abs(n_new ** 2 - (n ** 2 + d ** 2)) <= 1e-12 * n_new ** 2
