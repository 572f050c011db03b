"""Pins for the oracle's bf16 rounding and AdamW step (CPU only).

Each check ties the oracle to something other than itself: hand-worked bit
patterns, a library routine (torch's CPU bf16 cast, torch.optim.AdamW),
closed forms (step one from zeroed state is sign(g); a constant gradient gives
a step of exactly lr at every t) and the figures printed in the nanochat
discussion ("Stuck at the optimizer after figuring out backward()", reply by
mira687).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from workloads import seed0_gaussian_256x1024

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# --------------------------------------------------------------------- bf16 RNE

@pytest.mark.parametrize("bits,expect", [
    (0x3F800000, 0x3F80),   # 1.0
    (0x3F808000, 0x3F80),   # 1 + 2^-8: tie, lower neighbour is even
    (0x3F818000, 0x3F82),   # tie, upper neighbour is even
    (0x3F808001, 0x3F81),   # just above the tie
    (0x3F807FFF, 0x3F80),   # just below the tie
    (0x7F7FFFFF, 0x7F80),   # largest finite rounds to +inf
    (0x80000000, 0x8000),   # -0
    (0x7F800000, 0x7F80),   # +inf
    (0xFF800000, 0xFF80),   # -inf
    (0x00000001, 0x0000),   # smallest subnormal rounds to +0
    (0x00008000, 0x0000),   # subnormal tie to even (0)
    (0x00018000, 0x0002),   # subnormal tie to even (2)
    (0x00010000, 0x0001),   # exact subnormal bf16
])
def test_bf16_rne_hand_cases(bits, expect):
    x = np.array([bits], dtype=np.uint32).view(np.float32)
    assert int(O.f32_to_bf16_bits(x)[0]) == expect


def test_bf16_nan_stays_nan():
    x = np.array([0x7FC00000, 0x7F800001, 0xFFFFFFFF], dtype=np.uint32).view(np.float32)
    y = O.bf16_bits_to_f32(O.f32_to_bf16_bits(x))
    assert np.all(np.isnan(y))


def test_bf16_matches_torch_cpu_cast():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    ours = O.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(np.isnan(O.bf16_bits_to_f32(ours[nan])))


def test_bf16_roundtrip_exact_on_bf16_values():
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    x = O.bf16_bits_to_f32(h)
    back = O.f32_to_bf16_bits(x)
    keep = ~np.isnan(x)
    assert np.array_equal(back[keep], h[keep])


# --------------------------------------------------------------------- AdamW

def _cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def test_adamw_step1_is_sign_of_gradient_page_figures(golden_dir):
    """Step one from zeroed state moves each weight by lr*sign(g) (to eps)."""
    ref = json.load(open(os.path.join(golden_dir, "nanochat_discussion_measurements.json")))
    fig = ref["adamw_step1_seed0"]
    G = seed0_gaussian_256x1024().numpy()
    lr = 1.0
    p, m, v = O.adamw_step(np.zeros_like(G), G, np.zeros_like(G), np.zeros_like(G), 1,
                           lr=lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0)
    u = -p / lr
    assert round(float(np.mean(np.abs(u))), 4) == fig["abs_update"]
    assert round(_cos(u, np.sign(G)), 6) == fig["cos_vs_sign_G"]
    assert round(_cos(u, G), 3) == fig["cos_vs_G"]
    # the statistic itself: E|g| / sqrt(E g^2) = sqrt(2/pi) for a Gaussian
    assert abs(_cos(np.sign(G), G) - math.sqrt(2 / math.pi)) < 2e-3


def test_adamw_step1_eps0_exactly_lr():
    rng = np.random.default_rng(5)
    g = rng.standard_normal(4096).astype(np.float32) * 1e-3
    lr = 3e-4
    p, _, _ = O.adamw_step(np.zeros_like(g), g, np.zeros_like(g), np.zeros_like(g), 1,
                           lr=lr, beta1=0.9, beta2=0.95, eps=0.0, weight_decay=0.0)
    np.testing.assert_allclose(np.abs(p), lr, rtol=4e-7)
    assert np.array_equal(np.sign(p), -np.sign(g))


@pytest.mark.parametrize("b1,b2", [(0.9, 0.95), (0.8, 0.999), (0.5, 0.5)])
def test_adamw_constant_gradient_step_is_lr_every_step(b1, b2):
    """With full bias correction a constant g gives a step of exactly lr*sign(g)
    at every t, whatever the betas (exercise 3(b) of '3.9 Optimizers')."""
    g = np.array([2.0, -0.5, 1e-3, -7.0], dtype=np.float32)
    p = np.zeros(4, np.float32)
    m = np.zeros(4, np.float32)
    v = np.zeros(4, np.float32)
    lr = 1e-2
    for t in range(1, 8):
        p_new, m, v = O.adamw_step(p, g, m, v, t, lr=lr, beta1=b1, beta2=b2, eps=0.0,
                                   weight_decay=0.0)
        np.testing.assert_allclose(p_new - p, -lr * np.sign(g), rtol=2e-5)
        p = p_new


def test_adamw_zero_gradient_is_pure_decay():
    p = np.array([1.0, -2.0, 0.5], np.float32)
    z = np.zeros(3, np.float32)
    lr, wd = 0.125, 0.5
    p2, m2, v2 = O.adamw_step(p, z, z, z, 3, lr=lr, weight_decay=wd)
    assert np.array_equal(p2, p * np.float32(1 - lr * wd))
    assert not np.any(m2) and not np.any(v2)


@pytest.mark.parametrize("b1,b2,eps,wd,lr", [
    (0.9, 0.95, 1e-8, 0.1, 1e-3),
    (0.8, 0.95, 1e-8, 0.0, 3e-4),
    (0.9, 0.999, 1e-6, 0.01, 2e-2),
])
def test_adamw_matches_torch_adamw_5_steps(b1, b2, eps, wd, lr):
    """Against torch.optim.AdamW on CPU, 5 steps (page test: 1e-5; here 1e-6)."""
    gen = torch.Generator().manual_seed(7)
    p0 = torch.randn(3000, generator=gen) * 0.02
    grads = [torch.randn(3000, generator=gen) * 1e-3 for _ in range(5)]
    tp = torch.nn.Parameter(p0.clone())
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                            foreach=False)
    p = p0.numpy().copy()
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    for t, g in enumerate(grads, start=1):
        tp.grad = g.clone()
        opt.step()
        p, m, v = O.adamw_step(p, g.numpy(), m, v, t, lr=lr, beta1=b1, beta2=b2, eps=eps,
                               weight_decay=wd)
        ref = tp.detach().numpy()
        assert np.max(np.abs(p - ref)) <= 1e-6 * np.max(np.abs(ref))
    st = opt.state[tp]
    # torch forms the first moment with lerp: same value, different roundings
    em, ev = st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()
    assert np.max(np.abs(m - em)) <= 1e-6 * np.max(np.abs(em))
    assert np.max(np.abs(v - ev)) <= 1e-6 * np.max(np.abs(ev))


def test_adamw_planted_mistake_is_caught():
    """Dropping the bias correction (a plausible mistake) breaks the step-1 pin."""
    g = np.array([1.0, -1.0], np.float32)
    z = np.zeros(2, np.float32)
    p, m, v = O.adamw_step(z, g, z, z, 1, lr=1.0, eps=0.0, weight_decay=0.0)
    assert np.allclose(-p, np.sign(g))
    k = O.adamw_scalars(1.0, 0.9, 0.95, 0.0, 0.0, 1)
    uncorrected = (k["c1"] * g) / np.sqrt(k["c2"] * g * g)   # no bias correction
    assert not np.allclose(uncorrected, np.sign(g), rtol=0.1)
