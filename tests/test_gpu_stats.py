"""GPU parity of ma_muon_step_stats: the per-matrix ||W_new - W_old||_F and
||W_old||_F it reports, and the weights it writes (identical to ma_muon_step).

* ||W_old|| must match the oracle's norm of the same input weights, and
  ||W_new - W_old|| the norm of the change the kernel actually stored, to the
  fp32 summation bound (1e-5 relative).
* ||W_new - W_old|| must match the oracle's step: to 1e-3 with ns_steps = 0
  (the update is X0, whose bf16 rounding can differ in a few elements: the
  kernels normalise in fp32, the oracle in float64) and to the bf16
  iteration's bar of 2e-2 with five steps. The step is c_lr U plus the masked
  decay c_wd W, so | ||dW_gpu|| - ||dW_oracle|| | <= c_lr ||U_gpu - U_oracle||
  + c_wd ||W|| over the elements where the cautious masks differ; the first
  term is within 2e-2 of c_lr ||U|| by the iteration's bar, and the second is
  below 1e-5 of the step here (c_wd |W| ~ 4e-6 against steps ~ 1e-3, on the
  few elements where u w changes sign). Rounding W_new to bf16 changes the
  norm only to second order (about (2^-9 |W| / |dW|)^2 ~ 1e-3 relative).
Shapes cover the vector path (rows a multiple of 8) and the tile path (odd
columns), bf16 and fp32 weights, wide, square and tall matrices.

A step with stats applies the update in its own pass; a plain step applies it
in the epilogue of the last Newton-Schulz product wherever the weights allow
(bf16, rows a multiple of 8 elements, one stride between matrices): the
weights both write must be the same bits.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import f32r, need_gpu, say, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}
SHAPES = [((256, 256), 3, "bf16"), ((37, 53), 2, "bf16"), ((300, 100), 2, "f32"), ((128, 512), 2, "f32"),
          ((520, 264), 2, "bf16"), ((136, 392), 3, "bf16")]


def _groups(seed):
    gen = torch.Generator().manual_seed(seed)
    host, dev = [], []
    for (R, C), n, pdt in SHAPES:
        W = (torch.randn(n, R, C, generator=gen) * 0.02).to(TDT[pdt])
        G = (torch.randn(n, R, C, generator=gen) * 1e-3).to(torch.bfloat16)
        M = (torch.randn(n, R, C, generator=gen) * 3e-3).to(torch.bfloat16)
        host.append(tuple(to_np(t) for t in (W, G, M)) + (pdt,))
        dev.append([t.to(DEV) for t in (W, G, M)])
    return host, dev


def _hp(M, ns_steps):
    return M.MuonHParams(lr=f32r(0.02), momentum=f32r(0.95), weight_decay=f32r(0.01), nesterov=True,
                         ns_steps=ns_steps, coeffs=M.KELLER_JORDAN, cautious=True, equilibrate="pre",
                         ns_precision="bf16", norm_eps=f32r(1e-7), eq_eps=f32r(1e-7))


def _oracle(W, G, Mo, pdt, hp, ns_steps):
    return O.muon_step(W, G, Mo, lr=hp.lr, momentum=hp.momentum, coeffs=O.KELLER_JORDAN, ns_steps=ns_steps,
                       weight_decay=hp.weight_decay, cautious=True, equilibrate="pre", precision="bf16",
                       param_dtype=pdt, mom_dtype="bf16", norm_eps=hp.norm_eps, eq_eps=hp.eq_eps)


def _run(ns_steps, seed, with_stats=True):
    import adamw_optimizer_step_amd as M
    host, dev = _groups(seed)
    groups = [M.MuonGroup(*d) for d in dev]
    hp = _hp(M, ns_steps)
    total = sum(g.count for g in groups)
    stats = torch.full((2 * total,), float("nan"), dtype=torch.float32, device=DEV)
    M.muon_step(groups, hp, stats=stats if with_stats else None)
    torch.cuda.synchronize()
    return host, dev, hp, to_np(stats).reshape(total, 2)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("ns_steps,tol", [(0, 1e-3), (5, 2e-2)])
def test_stats_against_the_oracle(ns_steps, tol):
    say("stats: ns_steps", ns_steps)
    host, dev, hp, st = _run(ns_steps, seed=11 + ns_steps)
    k, worst = 0, 0.0
    for (W, G, Mo, pdt), d in zip(host, dev):
        for i in range(W.shape[0]):
            r = _oracle(W[i], G[i], Mo[i], pdt, hp, ns_steps)
            got = to_np(d[0][i])
            dn_own, wn = O.update_norms(W[i], got)       # the change the kernel stored
            dn_ora, _ = O.update_norms(W[i], r["W"])     # the oracle's change
            assert np.isfinite(st[k]).all(), (k, st[k])
            assert abs(st[k, 1] - wn) <= 1e-5 * wn, (k, st[k], wn)
            assert abs(st[k, 0] - dn_own) <= 1e-5 * dn_own, (k, st[k], dn_own)
            assert abs(st[k, 0] - dn_ora) <= tol * dn_ora, (k, st[k], dn_ora)
            worst = max(worst, abs(st[k, 0] - dn_ora) / dn_ora)
            k += 1
    say("stats: largest relative step-norm difference from the oracle", f"{worst:.2e}")


def test_stats_step_writes_the_same_weights():
    say("stats: same weights as the plain step")
    _, dev_a, _, _ = _run(5, seed=13, with_stats=True)
    _, dev_b, _, _ = _run(5, seed=13, with_stats=False)
    for a, b in zip(dev_a, dev_b):
        for x, y in zip(a[:2], b[:2]):
            iv = torch.int16 if x.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(x.view(iv), y.view(iv))


def test_stats_full_size_12_layer_d1024():
    """The 12-layer d=1024 parameter set (48 x 1024^2, 12 x 4096x1024,
    12 x 1024x4096) in one call: the first and last matrix of every group
    checked against the change actually stored; every value finite."""
    import adamw_optimizer_step_amd as M
    from workloads import materialize, workload
    wl = workload("c3_12L_d1024")
    say("stats: 12-layer d=1024 inputs")
    data = materialize(wl.scaled(adamw_segments=()), device=DEV, seed=2)
    picks = [(gi, k) for gi, d in enumerate(data["muon"]) for k in sorted({0, d["W"].shape[0] - 1})]
    before = {(gi, k): to_np(data["muon"][gi]["W"][k]) for gi, k in picks}
    groups = [M.MuonGroup(d["W"], d["G"], d["M"]) for d in data["muon"]]
    hp = M.MuonHParams(lr=wl.lr, momentum=wl.momentum, weight_decay=wl.weight_decay, nesterov=wl.nesterov,
                       ns_steps=wl.ns_steps, coeffs=M.KELLER_JORDAN, cautious=wl.cautious,
                       equilibrate=wl.equilibrate, ns_precision=wl.ns_precision)
    total = sum(g.count for g in groups)
    stats = torch.full((2 * total,), float("nan"), dtype=torch.float32, device=DEV)
    say("stats: 12-layer d=1024 step")
    M.muon_step(groups, hp, stats=stats)
    torch.cuda.synchronize()
    st = to_np(stats).reshape(total, 2)
    assert np.isfinite(st).all() and (st > 0).all()
    base = np.cumsum([0] + [g.count for g in groups])
    for gi, k in picks:
        dn, wn = O.update_norms(before[(gi, k)], to_np(data["muon"][gi]["W"][k]))
        row = st[base[gi] + k]
        assert abs(row[0] - dn) <= 1e-5 * dn and abs(row[1] - wn) <= 1e-5 * wn, (gi, k, row, dn, wn)
    del data, groups
    torch.cuda.empty_cache()
