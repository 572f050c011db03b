"""Pins of the Lion oracle (oracle/lion.py) against what the pages fix.

Sources: "3.9 Optimizers: SGD, Adam, Adafactor, Lion, Muon & Shampoo",
section "Lion: Learning the Sign of the Update" and exercise 5; "Muon vs
AdamW, Lion and Sophia: a fair race", section "Lion" (including the test it
describes: with no decay, three single steps each move every weight by the
learning rate, up or down, or not at all where gradient and momentum are zero).
"""
import json
import os

import numpy as np

import oracle as O

f32 = np.float32


def _num(v):
    if v is None:
        return None
    if isinstance(v, str):
        if v in ("nan", "inf", "-inf"):
            return float(v)
        if v == "-0":
            return -0.0
        return float.fromhex(v)
    return float(v)


def _same(a, e):
    a = f32(a)
    e = f32(e)
    if np.isnan(e):
        return bool(np.isnan(a))
    return a.view(np.uint32) == e.view(np.uint32)


def test_lion_hand_cases(golden_dir):
    doc = json.load(open(os.path.join(golden_dir, "lion_cases.json")))
    for c in doc["cases"]:
        hp = doc["sets"][c["set"]]
        p2, m2 = O.lion_step(f32([_num(c["p"])]), f32([_num(c["g"])]), f32([_num(c["m"])]), hp["lr"],
                             hp["beta1"], hp["beta2"], hp["weight_decay"])
        assert _same(p2[0], _num(c["p2"])), (c, p2[0])
        if c["m2"] is not None:
            assert _same(m2[0], _num(c["m2"])), (c, m2[0])


def test_each_weight_moves_by_lr_or_not_at_all():
    """The pages' own check: no decay, three steps one at a time; weights on a
    grid of 2^-6 and lr = 2^-10, so p -+ lr is exact and the move is exactly lr."""
    rng = np.random.default_rng(5)
    n = 4096
    lr = 2.0 ** -10
    p = f32(rng.integers(-128, 129, n) / 64.0)
    m = np.zeros(n, f32)
    dead = rng.random(n) < 0.1
    for _ in range(3):
        g = f32(rng.standard_normal(n))
        g[dead] = 0.0
        p2, m2 = O.lion_step(p, g, m, lr, 0.95, 0.98, 0.0)
        d = np.abs(p2.astype(np.float64) - p.astype(np.float64))
        assert np.all(d[~dead] == lr)
        assert np.array_equal(p2[dead].view(np.uint32), p[dead].view(np.uint32))
        assert np.all(m2[dead] == 0.0)
        p, m = p2, m2


def test_direction_and_momentum_in_exact_integer_arithmetic():
    """beta1 = 3/4, beta2 = 7/8, m = a/256, g = b/256 with small integers a, b:
    the blend is (3a + b)/1024 and the new momentum (7a + b)/2048 exactly, so
    the step's direction and the stored momentum follow from integers alone."""
    rng = np.random.default_rng(9)
    n = 20000
    a = rng.integers(-256, 257, n)
    b = rng.integers(-256, 257, n)
    lr = 2.0 ** -12
    p = f32(rng.integers(-512, 513, n) / 256.0)
    p2, m2 = O.lion_step(p, f32(b / 256.0), f32(a / 256.0), lr, 0.75, 0.875, 0.0)
    step = (p2.astype(np.float64) - p.astype(np.float64)) / lr
    assert np.array_equal(step, -np.sign(3 * a + b).astype(np.float64))
    assert np.array_equal(m2.astype(np.float64) * 2048.0, (7 * a + b).astype(np.float64))
    # the beta2 blend would point elsewhere on a good share of these entries
    assert np.mean(np.sign(3 * a + b) != np.sign(7 * a + b)) > 0.05


def test_constant_gradient_closed_form():
    """m0 = 0 and a constant gradient g: the momentum keeps g's sign, so every
    step subtracts lr*sign(g) after the decay, and
        p_t = cd^t p0 - lr sign(g) (1 - cd^t) / (1 - cd),   cd = 1 - lr*wd,
        m_t = (1 - beta2^t) g."""
    rng = np.random.default_rng(2)
    n = 1000
    lr, wd, b1, b2, T = 1e-3, 0.1, 0.95, 0.98, 25
    p0 = f32(rng.standard_normal(n))
    g = f32(rng.standard_normal(n) * 1e-2)
    p, m = p0.copy(), np.zeros(n, f32)
    for _ in range(T):
        p, m = O.lion_step(p, g, m, lr, b1, b2, wd)
    cd = 1.0 - float(f32(lr)) * float(f32(wd))
    s = np.sign(g.astype(np.float64))
    p_exact = cd ** T * p0.astype(np.float64) - float(f32(lr)) * s * (1.0 - cd ** T) / (1.0 - cd)
    m_exact = (1.0 - float(f32(b2)) ** T) * g.astype(np.float64)
    u = 2.0 ** -24
    assert np.all(np.abs(p - p_exact) <= 4 * T * u * (np.abs(p_exact) + T * lr))
    assert np.all(np.abs(m - m_exact) <= 4 * T * u * np.abs(g))


def test_sign_function():
    c = f32([2.0, -3.0, 0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45])
    s = O.lion.sign(c)
    assert np.array_equal(s[:6], f32([1, -1, 0, 0, 1, -1]))
    assert s[2].view(np.uint32) == 0 and s[3].view(np.uint32) == 0
    assert np.isnan(s[6])
    assert s[7] == 1 and s[8] == -1       # subnormal blends still count
