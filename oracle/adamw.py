"""AdamW step, per element, in binary32 with a fixed operation order (oracle).

Source: "3.9 Optimizers: SGD, Adam, Adafactor, Lion, Muon & Shampoo", section
"Implementing AdamW from scratch" (decay first, then the two moment updates,
bias corrections folded into the step size and the denominator, then
addcdiv), and "Chapter 4: The MuonAdamW Optimizer", section "The AdamW Step"
(same rule, moments written as lerp; the two forms agree in exact arithmetic).

Precision contract (the reading taken here, since the pages give the rule in
exact arithmetic only):

* scalars that depend on the hyperparameters and the step count are computed
  once in float64 and rounded to binary32:
  ``cd = 1 - lr*wd``, ``c1 = 1 - beta1``, ``c2 = 1 - beta2``,
  ``ss = lr / (1 - beta1**t)``, ``s2 = sqrt(1 - beta2**t)``;
* per element, every operation is one correctly rounded binary32 operation, no
  fused multiply-add:

      p   = p * cd                      (only when wd != 0)
      m   = beta1*m + c1*g
      v   = beta2*v + c2*(g*g)
      den = sqrt(v) / s2 + eps
      p   = p - ss * (m / den)
"""
import math

import numpy as np

f32 = np.float32


def adamw_scalars(lr, beta1, beta2, eps, weight_decay, step):
    """Step-dependent scalars (float64 on the host, then one rounding to fp32)."""
    t = int(step)
    if t < 1:
        raise ValueError("AdamW step count is 1-based")
    return {
        "cd": f32(1.0 - lr * weight_decay),
        "b1": f32(beta1),
        "b2": f32(beta2),
        "c1": f32(1.0 - beta1),
        "c2": f32(1.0 - beta2),
        "ss": f32(lr / (1.0 - beta1 ** t)),
        "s2": f32(math.sqrt(1.0 - beta2 ** t)),
        "eps": f32(eps),
        "decay": weight_decay != 0.0,
    }


def adamw_step(p, g, m, v, step, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1):
    """One AdamW step on flat fp32 arrays; returns new ``(p, m, v)`` (copies).

    ``step`` is the 1-based step count after increment (the first call passes 1).
    """
    k = adamw_scalars(lr, beta1, beta2, eps, weight_decay, step)
    p = np.array(p, dtype=f32, copy=True)
    g = np.asarray(g, dtype=f32)
    m = np.array(m, dtype=f32, copy=True)
    v = np.array(v, dtype=f32, copy=True)
    with np.errstate(all="ignore"):
        if k["decay"]:
            p = p * k["cd"]
        m = k["b1"] * m + k["c1"] * g
        v = k["b2"] * v + k["c2"] * (g * g)
        den = np.sqrt(v) / k["s2"] + k["eps"]
        p = p - k["ss"] * (m / den)
    return p.astype(f32), m.astype(f32), v.astype(f32)
