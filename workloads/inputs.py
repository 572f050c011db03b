"""Seeded synthetic inputs: parameter sets, gradients and optimizer state.

Every tensor is drawn from a seeded ``torch.Generator`` and only arranged into
shape here. The gradient recipes follow the workloads the pages describe:

* iid Gaussian gradients (the (256, 1024) experiment in the nanochat discussion
  "Stuck at the optimizer after figuring out backward()", reply by mira687);
* a rank-8-plus-noise gradient (same reply: a decaying spectrum, condition
  number in the hundreds);
* gradients with a prescribed singular spectrum, ``G = U diag(s) V^T`` with U, V
  Kronecker products of Haar-random orthogonal factors, so that singular
  vectors and values are known exactly to the tests.

No optimizer arithmetic (momentum, normalisation, polynomial steps, decay,
moment estimates) appears in this module.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import torch


# ----------------------------------------------------------------------------
# workload descriptions
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class MuonGroupSpec:
    """``count`` weight matrices of one shape ``rows x cols`` (row-major)."""
    name: str
    rows: int
    cols: int
    count: int


@dataclass(frozen=True)
class AdamWSegmentSpec:
    """One flat AdamW parameter buffer and its hyperparameters."""
    name: str
    numel: int
    lr: float = 3e-4
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.0


@dataclass(frozen=True)
class Workload:
    name: str
    muon_groups: Tuple[MuonGroupSpec, ...]
    adamw_segments: Tuple[AdamWSegmentSpec, ...] = ()
    # Muon hyperparameters (plain data; interpreted by the callers)
    lr: float = 0.02
    momentum: float = 0.95
    nesterov: bool = True
    ns_steps: int = 5
    weight_decay: float = 0.0
    cautious: bool = False
    equilibrate: str = "off"          # "off" | "pre" | "post"
    ns_precision: str = "bf16"        # "bf16" | "f32"
    lr_scale: str = "sqrt_max1_r_over_c"
    # storage types
    param_dtype: str = "bf16"
    grad_dtype: str = "bf16"
    mom_dtype: str = "bf16"
    # gradient recipe
    grad_kind: str = "gaussian"       # gaussian | spectrum_inv | lowrank16 | seed0 | rank8
    grad_rms: float = 1e-3
    mom_init: str = "gaussian"        # zero | gaussian
    adamw_step: int = 10              # 1-based step count used for AdamW state
    description: str = ""

    @property
    def muon_numel(self) -> int:
        return sum(g.rows * g.cols * g.count for g in self.muon_groups)

    @property
    def adamw_numel(self) -> int:
        return sum(s.numel for s in self.adamw_segments)

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def _layers(n_layers: int, d: int, mlp: int) -> Tuple[MuonGroupSpec, ...]:
    # per layer: Wq, Wk, Wv, Wo (d x d); c_fc (mlp x d, tall); c_proj (d x mlp, wide)
    return (
        MuonGroupSpec("attn_qkvo", d, d, 4 * n_layers),
        MuonGroupSpec("mlp_c_fc", mlp, d, n_layers),
        MuonGroupSpec("mlp_c_proj", d, mlp, n_layers),
    )


WORKLOADS: Dict[str, Workload] = {
    # single (256, 1024) fp32 matrix: the nanochat discussion's experiment
    "c1_256x1024_f32": Workload(
        name="c1_256x1024_f32",
        muon_groups=(MuonGroupSpec("c_proj", 256, 1024, 1),),
        lr=0.02, momentum=0.95, nesterov=True, ns_steps=5, weight_decay=0.0,
        cautious=False, equilibrate="off", ns_precision="f32",
        param_dtype="f32", grad_dtype="f32", mom_dtype="f32",
        grad_kind="seed0", mom_init="zero",
        description="one fp32 (256,1024) matrix, iid N(0,1) gradient from seed 0, "
                    "zero momentum, beta 0.95 Nesterov, 5 steps, lr 0.02, wd 0"),
    # 4-layer d=256 transformer parameter set
    "c2_4L_d256": Workload(
        name="c2_4L_d256",
        muon_groups=_layers(4, 256, 1024),
        adamw_segments=(
            AdamWSegmentSpec("wte", 32768 * 256, lr=3e-4, beta1=0.8, beta2=0.95),
            AdamWSegmentSpec("lm_head", 256 * 32768, lr=3e-4, beta1=0.8, beta2=0.95),
            AdamWSegmentSpec("scalars", 8, lr=3e-4, beta1=0.8, beta2=0.95),
        ),
        lr=0.02, weight_decay=0.0, cautious=False, equilibrate="off",
        grad_kind="spectrum_inv", grad_rms=1e-3,
        description="4L d=256: 16 x 256^2, 4 x 1024x256, 4 x 256x1024 via Muon (bf16); "
                    "wte 32768x256 + lm_head 256x32768 + 8 scalars via AdamW (0.8, 0.95)"),
    # 12-layer d=1024 parameter set: the headline workload
    "c3_12L_d1024": Workload(
        name="c3_12L_d1024",
        muon_groups=_layers(12, 1024, 4096),
        adamw_segments=(
            AdamWSegmentSpec("wte", 50304 * 1024, lr=3e-4, beta1=0.9, beta2=0.95),
            AdamWSegmentSpec("lm_head", 50304 * 1024, lr=3e-4, beta1=0.9, beta2=0.95),
        ),
        lr=0.02, weight_decay=0.01, cautious=True, equilibrate="pre",
        grad_kind="gaussian", grad_rms=1e-3,
        description="12L d=1024: 48 x 1024^2, 12 x 4096x1024, 12 x 1024x4096 via Muon "
                    "(bf16 W/G/momentum, cautious wd 0.01, MuonEq on); wte and lm_head "
                    "50304x1024 via AdamW in fp32"),
    # 24-layer d=2048 parameter set
    "c4_24L_d2048": Workload(
        name="c4_24L_d2048",
        muon_groups=_layers(24, 2048, 8192),
        adamw_segments=(AdamWSegmentSpec("wte", 65536 * 2048),),
        lr=0.02, weight_decay=0.01, cautious=True, equilibrate="pre",
        grad_kind="lowrank16", grad_rms=1e-3,
        description="24L d=2048: 96 x 2048^2, 24 x 8192x2048, 24 x 2048x8192 via Muon; "
                    "gradients rank 16 plus a 1e-3 floor (condition 1e3); AdamW on 65536x2048"),
    # 32-layer d=4096 matrices: the largest single-GPU share
    "c5_32L_d4096": Workload(
        name="c5_32L_d4096",
        muon_groups=_layers(32, 4096, 16384),
        lr=0.02, weight_decay=0.01, cautious=True, equilibrate="pre",
        grad_kind="spectrum_inv", grad_rms=1e-3,
        description="32L d=4096: 128 x 4096^2, 32 x 16384x4096 (tall), 32 x 4096x16384 "
                    "via Muon, power-law spectrum s_i ~ 1/i, no AdamW"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


# ----------------------------------------------------------------------------
# random draws
# ----------------------------------------------------------------------------

def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gaussian(shape, std: float, seed: int, device="cpu", dtype=torch.float32) -> torch.Tensor:
    g = _gen(seed, device)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def seed0_gaussian_256x1024() -> torch.Tensor:
    """``torch.manual_seed(0); torch.randn(256, 1024)`` (fp32, CPU)."""
    return torch.randn(256, 1024, generator=_gen(0))


def rank8_plus_noise_256x1024() -> torch.Tensor:
    """Rank-8 product plus 0.01 Gaussian noise, shape (256, 1024), seed 0."""
    g = _gen(0)
    a = torch.randn(256, 8, generator=g)
    b = torch.randn(8, 1024, generator=g)
    n = torch.randn(256, 1024, generator=g)
    return a @ b / math.sqrt(32.0) + 0.01 * n


def _split(n: int) -> Tuple[int, int]:
    """n = f1 * f2 with f1 the power of two nearest below sqrt(n) dividing n."""
    f1 = 1
    while (f1 * 2) * (f1 * 2) <= n and n % (f1 * 2) == 0:
        f1 *= 2
    return f1, n // f1


def _haar(rows: int, cols: int, g: torch.Generator) -> torch.Tensor:
    """rows x cols matrix with orthonormal columns (Haar measure), fp64 CPU."""
    z = torch.randn(rows, cols, generator=g, dtype=torch.float64)
    q, r = torch.linalg.qr(z)
    d = torch.sign(torch.diagonal(r))
    d[d == 0] = 1.0
    return q * d


def kron_spectrum_factors(rows: int, cols: int, kind: str, rms: float, seed: int):
    """Singular factors of a rows x cols gradient with a prescribed spectrum.

    Returns ``(U1, U2, V1, V2, s)`` (fp64, CPU) with ``U = kron(U1, U2)``
    (rows x m, orthonormal columns), ``V = kron(V1, V2)`` (cols x m) and ``s``
    (m,) such that ``G = U diag(s) V^T`` has entry RMS ``rms``.
    ``kind``: ``spectrum_inv`` (s_i = 1/i) or ``lowrank16`` (16 values at 1,
    the rest at 1e-3).
    """
    m = min(rows, cols)
    m1, m2 = _split(m)
    r1, r2 = _split(rows)
    c1, c2 = _split(cols)
    assert m1 <= min(r1, c1) and m2 <= min(r2, c2), (rows, cols)
    g = _gen(seed)
    U1, U2 = _haar(r1, m1, g), _haar(r2, m2, g)
    V1, V2 = _haar(c1, m1, g), _haar(c2, m2, g)
    i = torch.arange(1, m + 1, dtype=torch.float64)
    if kind == "spectrum_inv":
        s = 1.0 / i
    elif kind == "lowrank16":
        s = torch.full((m,), 1e-3, dtype=torch.float64)
        s[:16] = 1.0
    else:
        raise ValueError(kind)
    s = s * (rms * math.sqrt(rows * cols) / torch.linalg.vector_norm(s))
    return U1, U2, V1, V2, s


def kron_spectrum_matrix(factors, device="cpu", dtype=torch.float32) -> torch.Tensor:
    """Dense ``U diag(s) V^T`` from :func:`kron_spectrum_factors` output."""
    U1, U2, V1, V2, s = factors
    wd = torch.float64 if torch.device(device).type == "cpu" else torch.float32
    U = torch.kron(U1, U2).to(device=device, dtype=wd)
    V = torch.kron(V1, V2).to(device=device, dtype=wd)
    G = (U * s.to(device=device, dtype=wd)) @ V.t().contiguous()
    return G.to(dtype)


# ----------------------------------------------------------------------------
# materialisation
# ----------------------------------------------------------------------------

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def torch_dtype(name: str) -> torch.dtype:
    return _DT[name]


def _grad_group(wl: Workload, spec: MuonGroupSpec, gi: int, seed: int, device) -> torch.Tensor:
    R, C, n = spec.rows, spec.cols, spec.count
    dt = _DT[wl.grad_dtype]
    if wl.grad_kind == "seed0":
        assert (R, C, n) == (256, 1024, 1)
        return seed0_gaussian_256x1024().to(device=device, dtype=dt).reshape(1, R, C)
    if wl.grad_kind == "rank8":
        assert (R, C, n) == (256, 1024, 1)
        return rank8_plus_noise_256x1024().to(device=device, dtype=dt).reshape(1, R, C)
    if wl.grad_kind == "gaussian":
        return gaussian((n, R, C), wl.grad_rms, seed * 1000 + 17 * gi + 1, device, dt)
    out = torch.empty((n, R, C), device=device, dtype=dt)
    for k in range(n):
        out[k].copy_(kron_spectrum_matrix(grad_factors(wl, gi, k, seed), device=device))
    return out


def grad_factors(wl: Workload, gi: int, k: int, seed: int = 0):
    """Singular factors of matrix k of Muon group gi (prescribed-spectrum
    gradient kinds): the same ones :func:`materialize` builds it from."""
    spec = wl.muon_groups[gi]
    return kron_spectrum_factors(spec.rows, spec.cols, wl.grad_kind, wl.grad_rms, seed * 100003 + 7919 * gi + k)


def materialize(wl: Workload, device="cpu", seed: int = 0,
                groups: Optional[Sequence[int]] = None, max_count: Optional[int] = None) -> dict:
    """Build every tensor of workload ``wl`` on ``device``.

    Returns ``{"muon": [ {spec, W, G, M}, ... ], "adamw": [ {spec, p, g, m, v, step}, ... ]}``
    with Muon tensors stacked ``[count, rows, cols]`` (contiguous) and AdamW
    tensors flat fp32. ``groups`` restricts which Muon groups are built and
    ``max_count`` caps the matrices per group (for sampled checks).
    """
    out = {"muon": [], "adamw": []}
    for gi, spec in enumerate(wl.muon_groups):
        if groups is not None and gi not in groups:
            continue
        if max_count is not None and spec.count > max_count:
            spec = MuonGroupSpec(spec.name, spec.rows, spec.cols, max_count)
        R, C, n = spec.rows, spec.cols, spec.count
        W = gaussian((n, R, C), 0.02, seed * 1000 + 17 * gi + 2, device, _DT[wl.param_dtype])
        G = _grad_group(wl, spec, gi, seed, device)
        if wl.mom_init == "zero":
            M = torch.zeros((n, R, C), device=device, dtype=_DT[wl.mom_dtype])
        else:
            M = gaussian((n, R, C), 3.0 * wl.grad_rms, seed * 1000 + 17 * gi + 3, device,
                         _DT[wl.mom_dtype])
        out["muon"].append({"spec": spec, "W": W, "G": G, "M": M})
    for si, seg in enumerate(wl.adamw_segments):
        n = seg.numel
        base = seed * 1000 + 31 * si + 500
        p = gaussian((n,), 0.02, base + 1, device)
        g = gaussian((n,), 1e-3, base + 2, device)
        if wl.adamw_step <= 1:
            m = torch.zeros(n, device=device)
            v = torch.zeros(n, device=device)
        else:
            m = gaussian((n,), 3e-4, base + 3, device)
            v = gaussian((n,), 1e-3, base + 4, device).square_()
        out["adamw"].append({"spec": seg, "p": p, "g": g, "m": m, "v": v,
                             "step": max(1, wl.adamw_step)})
    return out
