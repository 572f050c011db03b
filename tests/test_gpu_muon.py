"""GPU parity of the Newton-Schulz iteration and the whole Muon step.

Tolerances (relative Frobenius error of the update U):
  bf16 iteration vs the oracle's bf16 rounding points  <= 2e-2
  fp32 iteration vs the oracle in float64              <= 1e-4
Stored momentum: bit-exact. Weights: both sides store
RNE((mask ? W - c_wd W : W) - c_lr U), so beyond one rounding step of W (and
c_wd |W| where the cautious masks differ) they may differ only through U: that
excess must stay within c_lr * tol * ||U||_F.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import bits_equal, f32r, first_mismatch, need_gpu, rel_fro, say, to_np, weight_excess
from workloads import materialize, rank8_plus_noise_256x1024, seed0_gaussian_256x1024, workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KJ = (3.4445, -4.7750, 2.0315)
TOL = {"bf16": 2e-2, "f32": 1e-4}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _x0(count, m, n, seed, dtype):
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn(count, m, n, generator=gen, dtype=torch.float64)
    x = x / torch.linalg.matrix_norm(x, keepdim=True)
    return x.to(dtype)


# --------------------------------------------------------------------- NS alone

@pytest.mark.parametrize("prec", ["bf16", "f32"])
@pytest.mark.parametrize("m,n,count", [(256, 1024, 1), (100, 300, 3), (1, 9, 2), (128, 128, 2),
                                       (256, 256, 4), (384, 640, 2), (1024, 1024, 1)])
@pytest.mark.parametrize("steps", [1, 5])
def test_newton_schulz_matches_oracle(prec, m, n, count, steps):
    import adamw_optimizer_step_amd as M
    dt = torch.bfloat16 if prec == "bf16" else torch.float32
    x0 = _x0(count, m, n, m * 31 + n + steps, dt)
    say("ns", prec, m, n, count, steps)
    u = to_np(M.newton_schulz(x0.to(DEV), KJ, steps))
    xs = to_np(x0).astype(np.float64)
    for k in range(count):
        ref = O.newton_schulz(xs[k], KJ, "bf16" if prec == "bf16" else "f64", steps)
        err = rel_fro(u[k], ref)
        assert err <= TOL[prec], (k, err)


def test_f32_tile_sizes_give_the_same_bits():
    """An fp32 launch with few jobs runs 64 x 64 tiles, a larger one 128 x 128.
    Both accumulate each output over k in the same order with the same MFMAs,
    so a 256 x 256 matrix iterated alone (3 Gram jobs at 128 x 128: the small
    tiles; K = 256 is not split) gives the bits it gets among 47 others (144
    Gram jobs: the large tiles); the large-tile launch also meets the fp32 bar."""
    import adamw_optimizer_step_amd as M
    x0 = _x0(48, 256, 256, 77, torch.float32)
    say("ns f32 tiles: 48 matrices of 256x256")
    many = to_np(M.newton_schulz(x0.to(DEV), KJ, 5))
    for k in (0, 47):
        say("ns f32 tiles: matrix", k, "alone")
        alone = to_np(M.newton_schulz(x0[k:k + 1].to(DEV), KJ, 5))[0]
        assert bits_equal(alone, many[k]), first_mismatch(alone, many[k])
    ref = O.newton_schulz(to_np(x0[47]).astype(np.float64), KJ, "f64", 5)
    assert rel_fro(many[47], ref) <= TOL["f32"]


@pytest.mark.parametrize("m,n,slices", [(256, 1024, 4), (100, 300, 2), (384, 640, 3)])
def test_f32_split_gram_matches_one_pass(m, n, slices):
    """A small fp32 launch splits its Gram product along K (here into `slices`
    slices of 256 columns) and adds the slices in order: the result differs
    from one pass over K by fp32 summation order only. The same matrices
    among enough others to take one pass must agree to 1e-5 relative, and
    both meet the fp32 bar against the oracle."""
    import adamw_optimizer_step_amd as M
    count = 3 if m == 100 else 1
    x0 = _x0(count, m, n, m + n + slices, torch.float32)
    say("ns f32 split gram:", m, n, count)
    split = to_np(M.newton_schulz(x0.to(DEV), KJ, 5))
    pad = _x0(64, m, n, 5, torch.float32)   # 64 more matrices: no longer a small launch
    one = to_np(M.newton_schulz(torch.cat([x0, pad]).to(DEV), KJ, 5))[:count]
    for k in range(count):
        assert rel_fro(split[k], one[k]) <= 1e-5, (k, rel_fro(split[k], one[k]))
        ref = O.newton_schulz(to_np(x0[k]).astype(np.float64), KJ, "f64", 5)
        assert rel_fro(split[k], ref) <= TOL["f32"]
        assert rel_fro(one[k], ref) <= TOL["f32"]


@pytest.mark.parametrize("m,n", [(256, 1024), (512, 512), (300, 700)])
def test_bf16_small_and_large_launches(m, n):
    """A bf16 Gram or POLY launch of fewer than 64 jobs of 256 x 256 runs the
    register-staged kernel (POLY adding b A in its epilogue, B stored with its
    mirrors); a larger one the LDS-DMA kernel (b A folded into the main loop,
    B stored as its upper triangle). The same matrices alone and among 64
    others (one launch of each form) both meet the bf16 bar against the
    oracle's rounding points, and each other's."""
    import adamw_optimizer_step_amd as M
    x0 = _x0(2, min(m, n), max(m, n), m + 3 * n, torch.bfloat16)
    say("ns bf16 small/large launch:", m, n)
    small = to_np(M.newton_schulz(x0.to(DEV), KJ, 5))
    pad = _x0(64, min(m, n), max(m, n), 9, torch.bfloat16)
    large = to_np(M.newton_schulz(torch.cat([x0, pad]).to(DEV), KJ, 5))[:2]
    for k in range(2):
        ref = O.newton_schulz(to_np(x0[k]).astype(np.float64), KJ, "bf16", 5)
        assert rel_fro(small[k], ref) <= TOL["bf16"], (k, rel_fro(small[k], ref))
        assert rel_fro(large[k], ref) <= TOL["bf16"], (k, rel_fro(large[k], ref))
        assert rel_fro(small[k], large[k]) <= TOL["bf16"], (k, rel_fro(small[k], large[k]))


@pytest.mark.parametrize("prec", ["bf16", "f32"])
def test_newton_schulz_special_coefficients(prec):
    """(1,0,0) copies X exactly; (0,1,0) gives X X^T X; (0,0,1) gives (X X^T)^2 X."""
    import adamw_optimizer_step_amd as M
    dt = torch.bfloat16 if prec == "bf16" else torch.float32
    x0 = _x0(2, 200, 520, 5, dt)
    xs = to_np(x0).astype(np.float64)
    say("ns special copy", prec)
    u = to_np(M.newton_schulz(x0.to(DEV), [(1.0, 0.0, 0.0)], 1))
    assert bits_equal(u, to_np(x0)), first_mismatch(u, to_np(x0))
    for co in [(0.0, 1.0, 0.0), (0.0, 0.0, 1.0), (0.5, -0.25, 0.125)]:
        say("ns special", co, prec)
        u = to_np(M.newton_schulz(x0.to(DEV), [co], 1))
        for k in range(2):
            ref = O.newton_schulz(xs[k], [co], "bf16" if prec == "bf16" else "f64")
            assert rel_fro(u[k], ref) <= TOL[prec], co


def test_newton_schulz_zero_steps_and_schedule():
    import adamw_optimizer_step_amd as M
    x0 = _x0(1, 64, 192, 9, torch.bfloat16)
    u = to_np(M.newton_schulz(x0.to(DEV), KJ, 0))
    assert bits_equal(u, to_np(x0))
    sched = [KJ, (2.0, -1.5, 0.5), (1.5, -0.5, 0.0), (15 / 8, -10 / 8, 3 / 8)]
    say("ns schedule")
    u = to_np(M.newton_schulz(x0.to(DEV), sched, 4))
    ref = O.newton_schulz(to_np(x0)[0].astype(np.float64), sched, "bf16")
    assert rel_fro(u[0], ref) <= TOL["bf16"]


@pytest.mark.parametrize("prec", ["bf16", "f32"])
@pytest.mark.parametrize("case", ["iid_256x1024", "rank8_256x1024", "iid_300x900", "iid_1024x1024"])
def test_newton_schulz_polar_express(prec, case):
    """The Polar Express table (a different triple per step, the first with
    large coefficients) against the oracle with the same table."""
    import adamw_optimizer_step_amd as M
    dt = torch.bfloat16 if prec == "bf16" else torch.float32
    if case == "rank8_256x1024":
        g = rank8_plus_noise_256x1024().double()
        x0 = (g / torch.linalg.matrix_norm(g)).unsqueeze(0).to(dt)
    else:
        m, n = (int(v) for v in case.split("_")[1].split("x"))
        x0 = _x0(2 if m < 1024 else 1, m, n, m + 7 * n, dt)
    table = list(M.POLAR_EXPRESS)
    say("ns polar express", prec, case)
    u = to_np(M.newton_schulz(x0.to(DEV), table, len(table)))
    xs = to_np(x0).astype(np.float64)
    for k in range(xs.shape[0]):
        ref = O.newton_schulz(xs[k], table, "bf16" if prec == "bf16" else "f64", len(table))
        assert rel_fro(u[k], ref) <= TOL[prec], (k, rel_fro(u[k], ref))


# --------------------------------------------------------------------- whole step

def _run_step(groups_np, hp, dts):
    """groups_np: list of (W, G, M) host float32 arrays [count, R, C]."""
    import adamw_optimizer_step_amd as M
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
    dev, mgs = [], []
    for W, G, Mo in groups_np:
        t = [torch.from_numpy(a).to(tdt[d]).to(DEV) for a, d in zip((W, G, Mo), dts)]
        dev.append(t)
        mgs.append(M.MuonGroup(*t))
    ws = M.muon_step(mgs, hp)
    torch.cuda.synchronize()
    return dev, mgs, ws


def _check_step(groups_np, dev, mgs, ws, hp, dts, sample=None):
    import adamw_optimizer_step_amd as M
    prec = hp.ns_precision
    for gi, ((W, G, Mo), (Wd, Gd, Md)) in enumerate(zip(groups_np, dev)):
        # stored momentum: bit-exact over every matrix
        m1, _ = O.momentum_stage(G, Mo, hp.momentum, hp.nesterov)
        em = O.round_to_bf16(m1) if dts[2] == "bf16" else m1
        got = to_np(Md)
        assert bits_equal(got, em), f"group {gi} momentum: {first_mismatch(got, em)}"
        ks = range(W.shape[0]) if sample is None else sample(W.shape[0])
        for k in ks:
            r = O.muon_step(W[k], G[k], Mo[k], lr=hp.lr, momentum=hp.momentum, nesterov=hp.nesterov,
                            coeffs=hp.coeffs, ns_steps=hp.ns_steps, weight_decay=hp.weight_decay,
                            cautious=hp.cautious, equilibrate=hp.equilibrate,
                            precision="bf16" if prec == "bf16" else "f64", param_dtype=dts[0],
                            mom_dtype=dts[2], norm_eps=hp.norm_eps, eq_eps=hp.eq_eps, lr_scale=hp.lr_scale)
            # the workspace holds the Newton-Schulz result (before any row scaling after it)
            u = to_np(M.muon_workspace_update(mgs, hp, ws, gi, k))
            err = rel_fro(u, r["U_ns"])
            assert err <= TOL[prec], f"group {gi} matrix {k}: update error {err:.3e}"
            w = to_np(Wd[k])
            excess = weight_excess(w, r["W"], W[k], r["c_wd"], dts[0] == "bf16")
            bound = float(r["c_lr"]) * TOL[prec] * float(np.linalg.norm(r["U"].astype(np.float64)))
            assert excess <= bound, f"group {gi} matrix {k}: weights {excess:.3e} > {bound:.3e}"


def _hp(**kw):
    import adamw_optimizer_step_amd as M
    d = dict(lr=f32r(0.02), momentum=f32r(0.95), weight_decay=0.0, nesterov=True, ns_steps=5,
             coeffs=KJ, cautious=False, equilibrate="off", ns_precision="bf16", norm_eps=f32r(1e-7),
             eq_eps=f32r(1e-7))
    d.update(kw)
    for k in ("weight_decay",):
        d[k] = f32r(d[k])
    return M.MuonHParams(**d)


@pytest.mark.parametrize("grad,steps", [("seed0", 1), ("seed0", 3), ("seed0", 5), ("rank8", 1),
                                        ("rank8", 3), ("rank8", 5)])
def test_single_fp32_matrix_256x1024(grad, steps):
    """One fp32 (256, 1024) matrix, zero momentum, beta 0.95 Nesterov, lr 0.02."""
    G = (seed0_gaussian_256x1024() if grad == "seed0" else rank8_plus_noise_256x1024()).numpy()[None]
    W = (torch.randn(1, 256, 1024, generator=torch.Generator().manual_seed(1)) * 0.02).numpy()
    Mo = np.zeros_like(G)
    hp = _hp(ns_precision="f32", ns_steps=steps)
    dts = ("f32", "f32", "f32")
    say("c1", grad, steps)
    dev, mgs, ws = _run_step([(W, G, Mo)], hp, dts)
    _check_step([(W, G, Mo)], dev, mgs, ws, hp, dts)
    # the same matrix through the bf16 path
    hp16 = _hp(ns_precision="bf16", ns_steps=steps)
    say("c1 bf16", grad, steps)
    dev, mgs, ws = _run_step([(W, G, Mo)], hp16, dts)
    _check_step([(W, G, Mo)], dev, mgs, ws, hp16, dts)


def _ragged_groups(dts):
    shapes = [(37, 53, 3), (300, 100, 2), (100, 300, 1), (1, 9, 2), (9, 1, 1), (128, 128, 2), (257, 255, 1)]
    rng = np.random.default_rng(77)
    groups_np = []
    for R, C, n in shapes:
        W = (rng.standard_normal((n, R, C)) * 0.02).astype(np.float32)
        G = (rng.standard_normal((n, R, C)) * 1e-3).astype(np.float32)
        Mo = (rng.standard_normal((n, R, C)) * 3e-3).astype(np.float32)
        if dts[0] == "bf16":
            W = O.round_to_bf16(W)
        if dts[1] == "bf16":
            G = O.round_to_bf16(G)
        if dts[2] == "bf16":
            Mo = O.round_to_bf16(Mo)
        groups_np.append((W, G, Mo))
    return groups_np


@pytest.mark.parametrize("eq", ["off", "pre", "post", "rms"])
@pytest.mark.parametrize("cautious,wd", [(False, 0.0), (True, 0.01)])
@pytest.mark.parametrize("dts", [("bf16", "bf16", "bf16"), ("f32", "f32", "f32"), ("f32", "bf16", "f32")])
def test_ragged_groups(eq, cautious, wd, dts):
    """Ragged, tall, wide, square and degenerate shapes in one call."""
    groups_np = _ragged_groups(dts)
    prec = "f32" if dts[0] == "f32" and dts[2] == "f32" else "bf16"
    extra = dict(eq_eps=f32r(1e-8), lr_scale="none") if eq == "rms" else {}
    hp = _hp(equilibrate=eq, cautious=cautious, weight_decay=wd, ns_precision=prec, **extra)
    say("ragged", eq, cautious, wd, dts)
    dev, mgs, ws = _run_step(groups_np, hp, dts)
    _check_step(groups_np, dev, mgs, ws, hp, dts)


@pytest.mark.parametrize("steps", [0, 5])
@pytest.mark.parametrize("dts", [("f32", "f32", "f32"), ("bf16", "bf16", "bf16"), ("bf16", "bf16", "f32"),
                                 ("bf16", "f32", "f32")])
def test_row_norms_of_long_rows(steps, dts):
    """MuonEq row factors for rows of one to seventeen 512-column chunks:
    1024 and 1536 columns (a wave per row, two and three of four chunk
    slots), 4608 and 8200 (four rows per wave in eight-chunk batches, the
    last partial), row counts that leave a block's four rows part empty, and a
    tall matrix whose rows are 1000 long (the second chunk partial). With no
    Newton-Schulz step the update is the row-scaled look-ahead itself, so a
    row sum that lost a chunk shows at the fp32 tolerance."""
    rng = np.random.default_rng(91)
    groups_np = []
    for R, C, n in [(20, 1024, 2), (7, 1536, 1), (5, 4608, 1), (3, 8200, 1), (1100, 1000, 1)]:
        W = (rng.standard_normal((n, R, C)) * 0.02).astype(np.float32)
        G = (rng.standard_normal((n, R, C)) * 1e-3).astype(np.float32)
        Mo = (rng.standard_normal((n, R, C)) * 3e-3).astype(np.float32)
        # one row far larger than the rest, one near zero
        G[:, 0, :] *= 50.0
        G[:, -1, :] *= 1e-3
        Mo[:, -1, :] *= 1e-3
        W, G, Mo = [O.round_to_bf16(a) if d == "bf16" else a for a, d in zip((W, G, Mo), dts)]
        groups_np.append((W, G, Mo))
    prec = "f32" if dts[0] == "f32" else "bf16"
    hp = _hp(equilibrate="pre", cautious=True, weight_decay=0.01, ns_precision=prec, ns_steps=steps,
             coeffs=KJ)
    say("long rows", steps, dts)
    dev, mgs, ws = _run_step(groups_np, hp, dts)
    if prec == "bf16" and steps > 0:
        # the 1024- and 1536-column groups take the one-pass form, the rest two passes
        import adamw_optimizer_step_amd as M
        assert [M.muon_row_pass(mgs, hp, i) for i in range(len(mgs))] == [True, True, False, False, False]
    _check_step(groups_np, dev, mgs, ws, hp, dts)


@pytest.mark.parametrize("scale", ["none", "sqrt_max1_r_over_c", "moonshot", "sqrt_max"])
@pytest.mark.parametrize("prec", ["bf16", "f32"])
def test_lr_scales(scale, prec):
    """The per-matrix lr multipliers the pages use, on ragged shapes."""
    dts = ("bf16", "bf16", "bf16") if prec == "bf16" else ("f32", "f32", "f32")
    groups_np = _ragged_groups(dts)
    hp = _hp(lr_scale=scale, cautious=True, weight_decay=0.01, ns_precision=prec)
    say("lr scale", scale, prec)
    dev, mgs, ws = _run_step(groups_np, hp, dts)
    _check_step(groups_np, dev, mgs, ws, hp, dts)


def test_zero_gradient_and_momentum():
    """G = 0 and M = 0: no NaN, the update is zero and only the decay acts."""
    W = np.full((2, 64, 96), 0.5, np.float32)
    Z = np.zeros_like(W)
    hp = _hp(weight_decay=0.25, ns_precision="f32")
    dts = ("f32", "f32", "f32")
    dev, mgs, ws = _run_step([(W, Z, Z)], hp, dts)
    w = to_np(dev[0][0])
    exp = np.float32(0.5) - np.float32(f32r(0.02) * 0.25) * np.float32(0.5)
    assert np.all(w == exp)


def test_step_is_deterministic():
    import adamw_optimizer_step_amd as M
    wl = workload("c2_4L_d256")
    outs = []
    for rep in range(2):
        data = materialize(wl, device=DEV, seed=3)
        mgs = [M.MuonGroup(d["W"], d["G"], d["M"]) for d in data["muon"]]
        hp = _hp(cautious=True, weight_decay=0.01, equilibrate="pre")
        M.muon_step(mgs, hp)
        torch.cuda.synchronize()
        outs.append([(d["W"].cpu(), d["M"].cpu()) for d in data["muon"]])
    for (w0, m0), (w1, m1) in zip(*outs):
        assert torch.equal(w0.view(torch.int16), w1.view(torch.int16))
        assert torch.equal(m0.view(torch.int16), m1.view(torch.int16))


def _workload_check(name, seed=0, max_count=None, sample_per_group=None, ns_steps=None, overlap=False):
    """One step of a workload: Muon then AdamW on one stream, or (overlap) the
    benchmark's launch, ma_muon_adamw_step with AdamW run by 256 lean
    workgroups on a second stream beside the Newton-Schulz products."""
    import adamw_optimizer_step_amd as M
    wl = workload(name)
    data = materialize(wl, device=DEV, seed=seed, max_count=max_count)
    host = [(to_np(d["W"]), to_np(d["G"]), to_np(d["M"])) for d in data["muon"]]
    hp = _hp(lr=f32r(wl.lr), momentum=f32r(wl.momentum), weight_decay=wl.weight_decay,
             nesterov=wl.nesterov, ns_steps=ns_steps or wl.ns_steps, cautious=wl.cautious,
             equilibrate=wl.equilibrate, ns_precision=wl.ns_precision)
    mgs = [M.MuonGroup(d["W"], d["G"], d["M"]) for d in data["muon"]]
    segs = []
    for a in data["adamw"]:
        s = a["spec"]
        segs.append(dict(param=a["p"], grad=a["g"], exp_avg=a["m"], exp_avg_sq=a["v"], step=a["step"],
                         lr=f32r(s.lr), beta1=f32r(s.beta1), beta2=f32r(s.beta2), eps=f32r(s.eps),
                         weight_decay=f32r(s.weight_decay)))
    before = [(to_np(a["p"]), to_np(a["g"]), to_np(a["m"]), to_np(a["v"])) for a in data["adamw"]]
    say("workload", name, [m.count for m in mgs], "overlapped" if overlap else "one stream")
    if overlap and segs:
        ws = M.optimizer_step(mgs, hp, segs, overlap=True, background_workgroups=256)
    else:
        ws = M.muon_step(mgs, hp)
        if segs:
            M.adamw_step(segs)
    torch.cuda.synchronize()
    dev = [(d["W"], d["G"], d["M"]) for d in data["muon"]]
    dts = (wl.param_dtype, wl.grad_dtype, wl.mom_dtype)
    sample = None
    if sample_per_group:
        sample = lambda n: sorted({0, n - 1, n // 2}) if sample_per_group >= 3 else sorted({0, n - 1})
    _check_step(host, dev, mgs, ws, hp, dts, sample=sample)
    # AdamW segments of the workload: bit-exact everywhere
    for (p, g, m, v), s in zip(before, segs):
        ep, em, ev = O.adamw_step(p, g, m, v, s["step"], lr=s["lr"], beta1=s["beta1"], beta2=s["beta2"],
                                  eps=s["eps"], weight_decay=s["weight_decay"])
        for got, exp in ((s["param"], ep), (s["exp_avg"], em), (s["exp_avg_sq"], ev)):
            got = to_np(got)
            assert bits_equal(got, exp), first_mismatch(got, exp)


def test_workload_4L_d256_full():
    _workload_check("c2_4L_d256")


def test_workload_12L_d1024_full_size_sampled():
    """The 12-layer d=1024 set at full size, launched as the benchmark times
    it: ma_muon_adamw_step, with AdamW on both 50304 x 1024 fp32 buffers by
    256 lean workgroups on a second stream beside the Newton-Schulz products.
    Momentum and AdamW are checked everywhere (bit-exact), updates and weights
    on three matrices per group."""
    _workload_check("c3_12L_d1024", sample_per_group=3, overlap=True)


def test_workload_24L_d2048_reduced_count():
    """Full-size 2048-wide matrices (rank-16 plus 1e-3 floor gradients), two per group."""
    _workload_check("c4_24L_d2048", max_count=2, sample_per_group=2)
