"""Lion step, per element, in binary32 with a fixed operation order (oracle).

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg.

Source: "3.9 Optimizers: SGD, Adam, Adafactor, Lion, Muon & Shampoo", section
"Lion: Learning the Sign of the Update" (the functional step) and its
exercise 5 (the same step as an optimizer class); "Muon vs AdamW, Lion and
Sophia: a fair race", section "Lion" (same rule: two betas, the sign of the
beta1 blend moves each weight by the learning rate, the momentum is updated
after the step with beta2 and the raw gradient, decay is lr times lambda).

Order of one step:

    p   = p * cd                         (cd = 1 - lr*wd, only when wd != 0)
    c   = beta1*m + c1*g                 (c1 = 1 - beta1; c is not stored)
    p   = p - lr * sign(c)
    m   = beta2*m + c2*g                 (c2 = 1 - beta2)

Precision contract (the pages state the rule in exact arithmetic only):

* ``cd``, ``c1``, ``c2`` are computed once in float64 from the binary32
  hyperparameters and rounded to binary32, as for AdamW;
* every per-element operation is one correctly rounded binary32 operation,
  no fused multiply-add;
* sign(c) is +1 for c > 0, -1 for c < 0, +0 for c = +0 or -0 and NaN for a NaN
  c, so a weight whose blend is zero keeps its exact bits (p - lr*0 = p for
  every p, -0 included) and a NaN blend makes the weight NaN.
"""
import numpy as np

f32 = np.float32


def lion_scalars(lr, beta1, beta2, weight_decay):
    """Binary32 scalars of one step (float64 on the host, one rounding each)."""
    lr, beta1, beta2, weight_decay = (float(f32(x)) for x in (lr, beta1, beta2, weight_decay))
    return {
        "lr": f32(lr),
        "cd": f32(1.0 - lr * weight_decay),
        "b1": f32(beta1),
        "b2": f32(beta2),
        "c1": f32(1.0 - beta1),
        "c2": f32(1.0 - beta2),
        "decay": weight_decay != 0.0,
    }


def sign(c):
    """+1, -1, +0 (for both zeros), NaN for NaN, elementwise, binary32."""
    c = np.asarray(c, dtype=f32)
    out = np.where(c > 0, f32(1.0), np.where(c < 0, f32(-1.0), f32(0.0))).astype(f32)
    return np.where(np.isnan(c), c, out).astype(f32)


def lion_step(p, g, m, lr, beta1=0.9, beta2=0.99, weight_decay=0.0):
    """One Lion step on flat fp32 arrays; returns new ``(p, m)`` (copies)."""
    k = lion_scalars(lr, beta1, beta2, weight_decay)
    p = np.array(p, dtype=f32, copy=True)
    g = np.asarray(g, dtype=f32)
    m = np.array(m, dtype=f32, copy=True)
    with np.errstate(all="ignore"):
        if k["decay"]:
            p = p * k["cd"]
        c = k["b1"] * m + k["c1"] * g
        p = p - k["lr"] * sign(c)
        m = k["b2"] * m + k["c2"] * g
    return p.astype(f32), m.astype(f32)
