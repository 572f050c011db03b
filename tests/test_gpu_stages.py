"""GPU parity, bit-exact stages: bf16 rounding, the AdamW step, the momentum
stage and the decay-and-update stage, each fed identical seeded inputs on both
sides and compared bit for bit with the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import bits_equal, f32r, first_mismatch, need_gpu, say, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


# --------------------------------------------------------------------- bf16 RNE

def test_bf16_round_structured_and_random():
    import adamw_optimizer_step_amd as M
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x4000, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xC000, 0xFFFF],
                    dtype=np.uint32)
    structured = (hi[:, None] | lows[None, :]).ravel()
    rnd = np.random.default_rng(11).integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    bits = np.concatenate([structured, rnd])
    x = bits.view(np.float32)
    say("bf16 round", x.size)
    out = M.bf16_round(torch.from_numpy(x.copy()).to(DEV)).cpu().numpy().view(np.uint16)
    ref = O.f32_to_bf16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(out[~nan], ref[~nan]), first_mismatch(
        O.bf16_bits_to_f32(out[~nan]), O.bf16_bits_to_f32(ref[~nan]))
    assert np.all(np.isnan(O.bf16_bits_to_f32(out[nan])))


# --------------------------------------------------------------------- AdamW

def _adamw_case(sizes, seed, step, wd, offset=0):
    rng = np.random.default_rng(seed)
    segs_np = []
    for i, n in enumerate(sizes):
        p = (rng.standard_normal(n) * 0.02).astype(np.float32)
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        if step == 1:
            m = np.zeros(n, np.float32)
            v = np.zeros(n, np.float32)
        else:
            m = (rng.standard_normal(n) * 3e-4).astype(np.float32)
            v = ((rng.standard_normal(n) * 1e-3) ** 2).astype(np.float32)
        # a few special values
        if n > 8:
            g[:4] = [0.0, -0.0, 1e-30, -3e-38]
            p[4] = -0.0
        hp = dict(lr=f32r(3e-4 * (i + 1)), beta1=f32r(0.9 if i % 2 == 0 else 0.8), beta2=f32r(0.95),
                  eps=f32r(1e-8), weight_decay=f32r(wd))
        segs_np.append((p, g, m, v, hp))
    return segs_np


@pytest.mark.parametrize("sizes,step,wd,offset", [
    ((1, 3, 4097, 100003), 1, 0.0, 0),
    ((1 << 20, 333, 8), 7, 0.1, 0),
    ((50000, 4096), 3, 0.01, 1),      # element offset 1: unaligned buffers, scalar path
    ((2,) * 30, 2, 0.1, 0),           # more segments than one launch holds
])
@pytest.mark.parametrize("workgroups", [None, 256, 3])
def test_adamw_bit_exact(sizes, step, wd, offset, workgroups):
    """ma_adamw_step, and ma_adamw_step_background with one workgroup per CU
    and with 3 workgroups striding over every block of every segment."""
    import adamw_optimizer_step_amd as M
    segs_np = _adamw_case(sizes, seed=len(sizes) * 31 + step, step=step, wd=wd)
    segs, keep = [], []
    for p, g, m, v, hp in segs_np:
        ts = []
        for a in (p, g, m, v):
            buf = torch.zeros(a.size + offset, dtype=torch.float32, device=DEV)
            buf[offset:].copy_(torch.from_numpy(a))
            keep.append(buf)
            ts.append(buf[offset:])
        segs.append(dict(param=ts[0], grad=ts[1], exp_avg=ts[2], exp_avg_sq=ts[3], step=step, **hp))
    say("adamw", sizes, step, wd, offset, workgroups)
    M.adamw_step(segs, workgroups=workgroups)
    torch.cuda.synchronize()
    for (p, g, m, v, hp), s in zip(segs_np, segs):
        ep, em, ev = O.adamw_step(p, g, m, v, step, **hp)
        for got, exp, name in ((s["param"], ep, "p"), (s["exp_avg"], em, "m"), (s["exp_avg_sq"], ev, "v")):
            got = to_np(got)
            assert bits_equal(got, exp), f"{name}: {first_mismatch(got, exp)}"


# --------------------------------------------------------------------- Muon momentum stage

def _group(shape, count, dts, seed, special=False):
    import adamw_optimizer_step_amd as M
    R, C = shape
    gen = torch.Generator().manual_seed(seed)
    W = (torch.randn(count, R, C, generator=gen) * 0.02).to(TDT[dts[0]])
    G = (torch.randn(count, R, C, generator=gen) * 1e-3).to(TDT[dts[1]])
    Mo = (torch.randn(count, R, C, generator=gen) * 3e-3).to(TDT[dts[2]])
    if special:
        G.view(-1)[:6] = torch.tensor([0.0, -0.0, float("inf"), 1e-40, -1e-39, 3e38]).to(G.dtype)
        Mo.view(-1)[:6] = torch.tensor([-0.0, 0.0, 1.0, 1e-40, 2e-39, 3e38]).to(Mo.dtype)
    host = (to_np(W), to_np(G), to_np(Mo))
    Wd, Gd, Md = W.to(DEV), G.to(DEV), Mo.to(DEV)
    return M.MuonGroup(Wd, Gd, Md), (Wd, Gd, Md), host


@pytest.mark.parametrize("shape", [(64, 64), (37, 53), (100, 300), (300, 100), (1, 9), (256, 1024)])
@pytest.mark.parametrize("dts", [("bf16", "bf16", "bf16"), ("f32", "f32", "f32"), ("bf16", "bf16", "f32"),
                                 ("f32", "bf16", "bf16")])
@pytest.mark.parametrize("nesterov", [True, False])
def test_momentum_stage_bit_exact(shape, dts, nesterov):
    import adamw_optimizer_step_amd as M
    seed = shape[0] * 1009 + shape[1] * 7 + sum(ord(ch) for ch in ''.join(dts))
    grp, dev, (W, G, Mo) = _group(shape, 3, dts, seed=seed, special=True)
    beta = f32r(0.95)
    say("momentum", shape, dts, nesterov)
    mt = M.momentum_stage(grp, beta, nesterov)
    torch.cuda.synchronize()
    m1, emt = O.momentum_stage(G, Mo, beta, nesterov)
    em = O.round_to_bf16(m1) if dts[2] == "bf16" else m1
    got_m = to_np(dev[2])
    assert bits_equal(got_m, em), first_mismatch(got_m, em)
    got_mt = to_np(mt)
    assert bits_equal(got_mt, emt), first_mismatch(got_mt, emt)


# --------------------------------------------------------------------- decay and update stage

@pytest.mark.parametrize("shape", [(64, 128), (37, 53), (300, 100), (1, 7), (1024, 1024)])
@pytest.mark.parametrize("pdt,udt", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32"), ("f32", "bf16")])
@pytest.mark.parametrize("cautious,decay", [(True, True), (False, True), (True, False)])
def test_update_stage_bit_exact(shape, pdt, udt, cautious, decay):
    import adamw_optimizer_step_amd as M
    R, C = shape
    grp, dev, (W, G, Mo) = _group(shape, 2, (pdt, "bf16", "bf16"), seed=R * 7 + C)
    gen = torch.Generator().manual_seed(R + 13 * C)
    U = (torch.randn(2, R, C, generator=gen) / np.sqrt(max(R, C))).to(TDT[udt])
    flat = U.view(-1)
    k = min(flat.numel(), 8)
    flat[:k] = torch.tensor([0.0, -0.0, float("nan"), float("inf"), -float("inf"), 1e-40, -5.0, 2.0][:k]).to(U.dtype)
    wf = dev[0].view(-1)
    wf[: min(4, wf.numel())] = torch.tensor([0.0, -0.0, 1.0, -1e-40][: min(4, wf.numel())]).to(wf.dtype)
    W = to_np(dev[0])
    u_np = to_np(U)
    c_lr = f32r(0.02 * np.sqrt(max(1.0, R / C)))
    c_wd = f32r(0.02 * np.sqrt(max(1.0, R / C)) * 0.01)
    say("update", shape, pdt, udt, cautious, decay)
    M.update_stage(grp, U.to(DEV).contiguous(), c_lr, c_wd, cautious, decay)
    torch.cuda.synchronize()
    w2, _ = O.post_stage(W, u_np, c_lr, c_wd, cautious, decay=decay)
    exp = O.round_to_bf16(w2) if pdt == "bf16" else w2
    got = to_np(dev[0])
    assert bits_equal(got, exp), first_mismatch(got, exp)
