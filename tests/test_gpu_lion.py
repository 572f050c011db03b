"""GPU parity of the Lion step: ma_lion_step against the oracle, bit for bit,
on seeded inputs (ragged and empty segments, unaligned buffers, more
segments than one launch holds, special values), over consecutive steps, and
on the hand-worked cases of tests/golden/lion_cases.json."""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import bits_equal, f32r, first_mismatch, need_gpu, say, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _case(sizes, seed, wd):
    rng = np.random.default_rng(seed)
    out = []
    for i, n in enumerate(sizes):
        p = (rng.standard_normal(n) * 0.02).astype(np.float32)
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        if n > 16:
            # zero blend from zero state, exact cancellation b1*m = -(1-b1)*g
            # (b1 = 1/2 on even segments), signed zeros, tiny, huge, inf, NaN
            g[:8] = [0.0, -0.0, 1e-30, -3e-38, np.inf, 2e-3, np.nan, 0.0]
            m[:8] = [0.0, 0.0, 0.0, 0.0, 0.0, -2e-3, 0.0, -0.0]
            p[:4] = [-0.0, 0.0, 3e38, -1e-3]
        hp = dict(lr=f32r(1e-4 * (i + 1)), beta1=f32r(0.5 if i % 2 == 0 else 0.95),
                  beta2=f32r(0.98 if i % 3 else 0.99), weight_decay=f32r(wd * (1 + i % 2)))
        out.append((p, g, m, hp))
    return out


def _to_dev(case, offset):
    segs, keep = [], []
    for p, g, m, hp in case:
        ts = []
        for a in (p, g, m):
            buf = torch.zeros(a.size + offset, dtype=torch.float32, device=DEV)
            buf[offset:].copy_(torch.from_numpy(a))
            keep.append(buf)
            ts.append(buf[offset:])
        segs.append(dict(param=ts[0], grad=ts[1], exp_avg=ts[2], **hp))
    return segs, keep


@pytest.mark.parametrize("sizes,wd,offset", [
    ((1, 3, 4097, 100003), 0.0, 0),
    ((1 << 20, 333, 8, 0), 1.0, 0),
    ((50000, 4096, 17), 0.3, 1),     # element offset 1: unaligned buffers, scalar path
    ((2,) * 30, 0.1, 0),             # more segments than one launch holds
    ((4096 * 3 + 5, 1023), 0.1, 3),
])
def test_lion_bit_exact(sizes, wd, offset):
    import adamw_optimizer_step_amd as M
    case = _case(sizes, seed=len(sizes) * 17 + offset, wd=wd)
    segs, keep = _to_dev(case, offset)
    say("lion", sizes, wd, offset)
    M.lion_step(segs)
    torch.cuda.synchronize()
    for (p, g, m, hp), s in zip(case, segs):
        ep, em = O.lion_step(p, g, m, **hp)
        for got, exp, name in ((s["param"], ep, "p"), (s["exp_avg"], em, "m")):
            got = to_np(got)
            assert bits_equal(got, exp), f"{name}: {first_mismatch(got, exp)}"


def test_lion_three_steps():
    """Three steps in a row with fresh gradients; state carried on both sides."""
    import adamw_optimizer_step_amd as M
    sizes = (300001, 4096, 7)
    case = _case(sizes, seed=77, wd=0.5)
    segs, keep = _to_dev(case, 0)
    rng = np.random.default_rng(78)
    state = [(p.copy(), m.copy()) for p, g, m, hp in case]
    for step in range(3):
        grads = [(rng.standard_normal(p.size) * 1e-3).astype(np.float32) for p, _, _, _ in case]
        for s, g in zip(segs, grads):
            s["grad"].copy_(torch.from_numpy(g))
        say("lion step", step)
        M.lion_step(segs)
        torch.cuda.synchronize()
        state = [O.lion_step(p, g, m, **hp) for (p, m), g, (_, _, _, hp) in zip(state, grads, case)]
        for (ep, em), s in zip(state, segs):
            for got, exp, name in ((s["param"], ep, "p"), (s["exp_avg"], em, "m")):
                got = to_np(got)
                assert bits_equal(got, exp), f"step {step} {name}: {first_mismatch(got, exp)}"


def _num(v):
    if isinstance(v, str):
        if v in ("nan", "inf", "-inf"):
            return float(v)
        return -0.0 if v == "-0" else float.fromhex(v)
    return float(v)


def test_lion_hand_cases_on_gpu():
    import adamw_optimizer_step_amd as M
    doc = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lion_cases.json")))
    for c in doc["cases"]:
        hp = doc["sets"][c["set"]]
        p = torch.tensor([_num(c["p"])] * 8, dtype=torch.float32, device=DEV)
        g = torch.tensor([_num(c["g"])] * 8, dtype=torch.float32, device=DEV)
        m = torch.tensor([_num(c["m"])] * 8, dtype=torch.float32, device=DEV)
        M.lion_step([dict(param=p, grad=g, exp_avg=m, lr=hp["lr"], beta1=hp["beta1"], beta2=hp["beta2"],
                          weight_decay=hp["weight_decay"])])
        torch.cuda.synchronize()
        exp_p = np.full(8, _num(c["p2"]), np.float32)
        assert bits_equal(to_np(p), exp_p), (c, to_np(p)[0])
        if c["m2"] is not None:
            assert bits_equal(to_np(m), np.full(8, _num(c["m2"]), np.float32)), (c, to_np(m)[0])
