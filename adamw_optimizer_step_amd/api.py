"""Thin Python binding of the Muon + AdamW library.

Argument marshalling only: torch supplies device memory, pointers and the
current HIP stream; every step of the optimizer runs in the HIP kernels of
``libmuon_adamw.so``. Names follow the C ABI (include/muon_adamw.h).
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Union

import torch

from . import _lib as L

# Keller Jordan's coefficient triple, repeated at every step ("Chapter 4: The
# MuonAdamW Optimizer", section "Polar Express: Newton-Schulz Orthogonalization").
KELLER_JORDAN = (3.4445, -4.7750, 2.0315)

_DT = {torch.bfloat16: L.MA_BF16, torch.float32: L.MA_F32}
_PREC = {"bf16": L.MA_BF16, "f32": L.MA_F32}
_EQ = {"off": L.MA_EQ_OFF, "pre": L.MA_EQ_ROWS_PRE, "post": L.MA_EQ_ROWS_POST, "rms": L.MA_EQ_ROWS_RMS}
_SCALE = {"none": L.MA_SCALE_NONE, "sqrt_max1_r_over_c": L.MA_SCALE_SQRT_MAX1_R_OVER_C,
          "moonshot": L.MA_SCALE_MOONSHOT, "sqrt_max": L.MA_SCALE_SQRT_MAX}


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)") from None


def _stream(device: torch.device, stream=None) -> Optional[int]:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream(device).cuda_stream


@dataclass
class MuonHParams:
    lr: float = 0.02
    momentum: float = 0.95
    weight_decay: float = 0.0
    nesterov: bool = True
    ns_steps: int = 5
    coeffs: Sequence = KELLER_JORDAN   # one (a, b, c) triple, or ns_steps triples
    cautious: bool = False
    equilibrate: str = "off"           # off | pre | post
    ns_precision: str = "bf16"         # bf16 | f32
    lr_scale: str = "sqrt_max1_r_over_c"
    norm_eps: float = 1e-7
    eq_eps: float = 1e-7
    check_finite: bool = False         # flag matrices with non-finite norms (see muon_nonfinite)

    def table(self) -> List[float]:
        c = list(self.coeffs)
        if len(c) == 3 and all(isinstance(v, (int, float)) for v in c):
            c = [tuple(c)] * self.ns_steps
        if len(c) != self.ns_steps:
            raise ValueError("coefficient table length must equal ns_steps")
        return [float(v) for t in c for v in t]

    def to_c(self):
        tab = self.table()
        arr = (C.c_float * max(1, len(tab)))(*tab)
        hp = L.MuonHParamsC(
            lr=self.lr, momentum=self.momentum, weight_decay=self.weight_decay,
            nesterov=int(bool(self.nesterov)), ns_steps=int(self.ns_steps),
            abc=C.cast(arr, C.POINTER(C.c_float)), cautious=int(bool(self.cautious)),
            equilibrate=_EQ[self.equilibrate], ns_precision=_PREC[self.ns_precision],
            lr_scale=_SCALE[self.lr_scale], norm_eps=self.norm_eps, eq_eps=self.eq_eps,
            check_finite=int(bool(self.check_finite)))
        return hp, arr


def _matrix_ptrs(x: Union[torch.Tensor, Sequence[torch.Tensor]], rows: int, cols: int) -> List[int]:
    if isinstance(x, torch.Tensor):
        if x.dim() == 2:
            x = x.unsqueeze(0)
        if x.dim() != 3 or tuple(x.shape[1:]) != (rows, cols) or not x.is_contiguous():
            raise ValueError(f"expected a contiguous [count, {rows}, {cols}] tensor, got {tuple(x.shape)}")
        step = rows * cols * x.element_size()
        return [x.data_ptr() + i * step for i in range(x.shape[0])]
    out = []
    for t in x:
        if tuple(t.shape) != (rows, cols) or not t.is_contiguous():
            raise ValueError(f"expected contiguous ({rows}, {cols}) matrices")
        out.append(t.data_ptr())
    return out


def _flat(x):
    if x is None:
        return []
    if isinstance(x, torch.Tensor):
        return [x]
    return [t for t in x if t is not None]


def _check_cuda(tensors, dev: torch.device, what: str):
    """Every tensor a launch reads or writes lives on the GPU `dev`: the
    library takes raw device pointers, so a host or other-GPU tensor would
    reach a kernel as a bad address."""
    if dev.type != "cuda":
        raise ValueError(f"{what}: expected CUDA tensors, got a tensor on {dev}")
    for t in tensors:
        if t.device != dev:
            raise ValueError(f"{what}: every tensor must be on {dev}, got one on {t.device}")


def _check_groups(groups) -> torch.device:
    dev = groups[0].device
    for g in groups:
        _check_cuda([t for x in g._keep for t in _flat(x)], dev, "Muon groups")
    return dev


def _check_dense(g):
    if g.layout != torch.strided:
        # as an optimizer's step() does for sparse gradients ("3.9 Optimizers",
        # section "Implementing AdamW from scratch")
        raise TypeError("sparse gradients are not supported")


def _as_list(x):
    if isinstance(x, torch.Tensor):
        return [x] if x.dim() == 2 else [x[i] for i in range(x.shape[0])]
    return list(x)


def _drop_missing(params, grads, momentum):
    """Matrices whose gradient is None are left out of the step (as an
    optimizer's step() skips parameters without a gradient, "3.9 Optimizers",
    section "Implementing AdamW from scratch"). Returns the kept params,
    grads and momentum and their indices."""
    if isinstance(grads, torch.Tensor):
        _check_dense(grads)
        return params, grads, momentum, list(range(1 if grads.dim() == 2 else grads.shape[0]))
    P, Mo = _as_list(params), _as_list(momentum)
    G = [None] * len(P) if grads is None else list(grads)
    if not (len(P) == len(G) == len(Mo)):
        raise ValueError("params, grads and momentum differ in count")
    keep = [i for i, g in enumerate(G) if g is not None]
    for i in keep:
        _check_dense(G[i])
    return [P[i] for i in keep], [G[i] for i in keep], [Mo[i] for i in keep], keep


class MuonGroup:
    """``count`` same-shape matrices: stacked ``[count, R, C]`` tensors or lists.

    A gradient of ``None`` (a list entry, or ``grads=None`` for the whole
    group) leaves that matrix out of the step: its weight and momentum are not
    touched. ``kept`` lists the indices that take part. Sparse gradients are
    rejected."""

    def __init__(self, params, grads, momentum):
        first = params if isinstance(params, torch.Tensor) else params[0]
        self.rows, self.cols = int(first.shape[-2]), int(first.shape[-1])
        self.device = first.device
        self.dtypes = tuple(_dt(t if isinstance(t, torch.Tensor) else t[0]) for t in (params, momentum))
        params, grads, momentum, self.kept = _drop_missing(params, grads, momentum)
        gd = grads if isinstance(grads, torch.Tensor) else (grads[0] if grads else None)
        self.dtypes = (self.dtypes[0], _dt(gd) if gd is not None else self.dtypes[0], self.dtypes[1])
        self.p = _matrix_ptrs(params, self.rows, self.cols)
        self.g = _matrix_ptrs(grads, self.rows, self.cols)
        self.m = _matrix_ptrs(momentum, self.rows, self.cols)
        if not (len(self.p) == len(self.g) == len(self.m)):
            raise ValueError("params, grads and momentum differ in count")
        self.count = len(self.p)
        self._keep = (params, grads, momentum)

    def to_c(self):
        n = self.count
        pa, ga, ma = (C.c_void_p * max(1, n))(*self.p), (C.c_void_p * max(1, n))(*self.g), (C.c_void_p * max(1, n))(*self.m)
        s = L.MuonGroupC(rows=self.rows, cols=self.cols, count=n, param_dtype=self.dtypes[0],
                         grad_dtype=self.dtypes[1], mom_dtype=self.dtypes[2],
                         params=C.cast(pa, C.POINTER(C.c_void_p)), grads=C.cast(ga, C.POINTER(C.c_void_p)),
                         momentum=C.cast(ma, C.POINTER(C.c_void_p)))
        return s, (pa, ga, ma)


def _groups_c(groups: Sequence[MuonGroup]):
    arr = (L.MuonGroupC * max(1, len(groups)))()
    keep = []
    for i, g in enumerate(groups):
        arr[i], k = g.to_c()
        keep.append(k)
    return arr, keep


def muon_workspace_size(groups: Sequence[MuonGroup], hp: MuonHParams) -> int:
    garr, keep = _groups_c(groups)
    h, tab = hp.to_c()
    n = L.lib().ma_muon_workspace_size(garr, len(groups), C.byref(h))
    if n == 0 and groups:
        L.check(L.MA_ERR_INVALID_ARG)
    return int(n)


def muon_step(groups: Sequence[MuonGroup], hp: MuonHParams, workspace: Optional[torch.Tensor] = None,
              stream=None, stats: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One Muon step over ``groups`` (in place). Returns the workspace used.

    With ``stats`` (contiguous fp32 tensor of at least 2 values per matrix,
    groups in order), each matrix's ||W_new - W_old||_F and ||W_old||_F are
    written to it (``ma_muon_step_stats``)."""
    if not groups:
        return workspace
    dev = _check_groups(groups)
    need = muon_workspace_size(groups, hp)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_cuda([workspace] + ([stats] if stats is not None else []), dev, "workspace and stats")
    garr, keep = _groups_c(groups)
    h, tab = hp.to_c()
    ws, st = C.c_void_p(workspace.data_ptr()), C.c_void_p(_stream(dev, stream))
    if stats is None:
        L.check(L.lib().ma_muon_step(garr, len(groups), C.byref(h), ws, workspace.numel(), st))
    else:
        total = sum(g.count for g in groups)
        if stats.dtype != torch.float32 or not stats.is_contiguous() or stats.numel() < 2 * total:
            raise ValueError(f"stats must be a contiguous fp32 tensor of at least {2 * total} values")
        L.check(L.lib().ma_muon_step_stats(garr, len(groups), C.byref(h), ws, workspace.numel(),
                                           C.c_void_p(stats.data_ptr()), st))
    return workspace


def muon_step_noalloc(groups: Sequence[MuonGroup], hp: MuonHParams, stream=None) -> None:
    """``muon_step`` without a workspace (``ma_muon_step_noalloc``): the
    library's fixed per-GPU scratch array stands in for it, so nothing is
    allocated. For steps whose workspace fits in MA_NOALLOC_SCRATCH_BYTES;
    calls that overlap on one GPU must be ordered by the caller."""
    if not groups:
        return
    dev = _check_groups(groups)
    garr, keep = _groups_c(groups)
    h, tab = hp.to_c()
    with torch.cuda.device(dev):   # the library's scratch array is the current device's
        L.check(L.lib().ma_muon_step_noalloc(garr, len(groups), C.byref(h), C.c_void_p(_stream(dev, stream))))


def muon_nonfinite(groups: Sequence[MuonGroup], hp: MuonHParams, workspace: torch.Tensor) -> List[bool]:
    """After a step with ``hp.check_finite`` (waits for the device): per matrix
    of ``groups`` (in order), whether its look-ahead momentum had non-finite
    norms, so that its weight was left unchanged (``ma_muon_nonfinite``)."""
    garr, keep = _groups_c(groups)
    h, tab = hp.to_c()
    total = sum(g.count for g in groups)
    flags = (C.c_int32 * max(1, total))()
    torch.cuda.synchronize(groups[0].device) if groups else None
    rc = L.lib().ma_muon_nonfinite(garr, len(groups), C.byref(h), C.c_void_p(workspace.data_ptr()), flags)
    if rc not in (L.MA_OK, L.MA_ERR_NONFINITE):
        L.check(rc)
    return [bool(flags[i]) for i in range(total)]


def muon_row_pass(groups: Sequence[MuonGroup], hp: MuonHParams, group: int) -> bool:
    """Whether ``muon_step`` reads group ``group``'s G and M once (momentum,
    MuonEq row sums and X0 in one pass, the Frobenius factor applied by the
    first Newton-Schulz products) rather than twice (``ma_muon_row_pass``)."""
    garr, keep = _groups_c(groups)
    h, tab = hp.to_c()
    rc = L.lib().ma_muon_row_pass(garr, len(groups), C.byref(h), group)
    if rc < 0:
        L.check(rc)
    return rc == 1


def muon_workspace_update(groups: Sequence[MuonGroup], hp: MuonHParams, workspace: torch.Tensor,
                          group: int, index: int) -> torch.Tensor:
    """View of the update U of one matrix inside ``workspace`` (parameter layout)."""
    garr, keep = _groups_c(groups)
    h, tab = hp.to_c()
    u, ld, tr, eb = C.c_void_p(), C.c_int64(), C.c_int32(), C.c_int32()
    L.check(L.lib().ma_muon_workspace_update(garr, len(groups), C.byref(h), C.c_void_p(workspace.data_ptr()),
                                             group, index, C.byref(u), C.byref(ld), C.byref(tr), C.byref(eb)))
    g = groups[group]
    off = u.value - workspace.data_ptr()
    dt = torch.bfloat16 if eb.value == 2 else torch.float32
    flat = workspace[off: off + g.rows * ld.value * eb.value].view(dt)
    return flat.view(g.rows, ld.value)[:, : g.cols]


def _adamw_c(segments: Sequence[dict]):
    # a segment whose gradient is None takes no step; sparse gradients are rejected
    segments = [s for s in segments if s["grad"] is not None]
    for s in segments:
        _check_dense(s["grad"])
    arr = (L.AdamWSegmentC * max(1, len(segments)))()
    for i, s in enumerate(segments):
        p, g, m, v = s["param"], s["grad"], s["exp_avg"], s["exp_avg_sq"]
        for t in (p, g, m, v):
            if not t.is_contiguous() or t.numel() != p.numel():
                raise ValueError("AdamW buffers must be contiguous and of equal size")
        arr[i] = L.AdamWSegmentC(param=p.data_ptr(), grad=g.data_ptr(), exp_avg=m.data_ptr(),
                                 exp_avg_sq=v.data_ptr(), n=p.numel(), param_dtype=_dt(p),
                                 grad_dtype=_dt(g), lr=s["lr"], beta1=s.get("beta1", 0.9),
                                 beta2=s.get("beta2", 0.95), eps=s.get("eps", 1e-8),
                                 weight_decay=s.get("weight_decay", 0.0), step=int(s["step"]))
    return arr, len(segments)


def adamw_step(segments: Sequence[dict], stream=None, workgroups: Optional[int] = None) -> None:
    """One AdamW step. Each segment: param, grad, exp_avg, exp_avg_sq (fp32
    tensors, contiguous), lr, beta1, beta2, eps, weight_decay, step (1-based).
    With ``workgroups``, the same update by that many persistent workgroups
    with a small register footprint (``ma_adamw_step_background``), for
    running beside the Newton-Schulz GEMMs on another stream."""
    if not segments:
        return
    arr, n = _adamw_c(segments)
    dev = segments[0]["param"].device
    _check_cuda([s[k] for s in segments if s["grad"] is not None for k in ("param", "grad", "exp_avg", "exp_avg_sq")],
                dev, "AdamW buffers")
    if workgroups is None:
        L.check(L.lib().ma_adamw_step(arr, n, C.c_void_p(_stream(dev, stream))))
    else:
        L.check(L.lib().ma_adamw_step_background(arr, n, int(workgroups), C.c_void_p(_stream(dev, stream))))


_SIDE = {}


def optimizer_step(groups: Sequence[MuonGroup], hp: MuonHParams, adamw_segments: Sequence[dict],
                   workspace: Optional[torch.Tensor] = None, overlap: bool = True,
                   background_workgroups: int = 256) -> torch.Tensor:
    """One MuonAdamW step: ``muon_step`` over ``groups`` and ``adamw_step``
    over ``adamw_segments`` (disjoint buffers), both ordered after the work
    already on the current stream, with everything done once the current
    stream reaches the end of the call. With ``overlap`` (``ma_muon_adamw_step``),
    AdamW runs on a second stream (default priority) by
    ``background_workgroups`` lean workgroups beside the Muon step's
    Newton-Schulz products, so that the HBM-bound update shares the GPU with
    the MFMA-bound iteration; the results are identical either way.
    Capturable in a HIP graph. Returns the Muon workspace."""
    if not adamw_segments or not groups:
        ws = muon_step(groups, hp, workspace=workspace) if groups else workspace
        adamw_step(adamw_segments)
        return ws
    if not overlap:
        ws = muon_step(groups, hp, workspace=workspace)
        adamw_step(adamw_segments)
        return ws
    dev = _check_groups(groups)
    need = muon_workspace_size(groups, hp)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_cuda([workspace] + [s[k] for s in adamw_segments if s["grad"] is not None
                               for k in ("param", "grad", "exp_avg", "exp_avg_sq")], dev, "workspace and AdamW buffers")
    side = _SIDE.get(dev)
    if side is None:
        side = _SIDE[dev] = torch.cuda.Stream(device=dev)
    garr, keep = _groups_c(groups)
    h, tab = hp.to_c()
    arr, n_seg = _adamw_c(adamw_segments)
    with torch.cuda.device(dev):   # the library's fork and join events are the current device's
        L.check(L.lib().ma_muon_adamw_step(garr, len(groups), C.byref(h), C.c_void_p(workspace.data_ptr()),
                                           workspace.numel(), arr, n_seg, int(background_workgroups),
                                           C.c_void_p(_stream(dev)), C.c_void_p(side.cuda_stream)))
    return workspace


def lion_step(segments: Sequence[dict], stream=None) -> None:
    """One Lion step. Each segment: param, grad, exp_avg (fp32 tensors,
    contiguous, equal sizes), lr, beta1, beta2, weight_decay."""
    if not segments:
        return
    arr = (L.LionSegmentC * len(segments))()
    dev = segments[0]["param"].device
    _check_cuda([s[k] for s in segments for k in ("param", "grad", "exp_avg")], dev, "Lion buffers")
    for i, s in enumerate(segments):
        p, g, m = s["param"], s["grad"], s["exp_avg"]
        for t in (p, g, m):
            if not t.is_contiguous() or t.numel() != p.numel():
                raise ValueError("Lion buffers must be contiguous and of equal size")
        arr[i] = L.LionSegmentC(param=p.data_ptr(), grad=g.data_ptr(), exp_avg=m.data_ptr(), n=p.numel(),
                                param_dtype=_dt(p), grad_dtype=_dt(g), lr=s["lr"], beta1=s.get("beta1", 0.9),
                                beta2=s.get("beta2", 0.99), weight_decay=s.get("weight_decay", 0.0))
    L.check(L.lib().ma_lion_step(arr, len(segments), C.c_void_p(_stream(dev, stream))))


# ---------------------------------------------------------------------------
# stage entry points (used by the tests)
# ---------------------------------------------------------------------------

def bf16_round(x: torch.Tensor, stream=None) -> torch.Tensor:
    _check_cuda([x], x.device, "bf16_round")
    out = torch.empty(x.numel(), dtype=torch.int16, device=x.device)
    L.check(L.lib().ma_test_bf16_round(C.c_void_p(x.data_ptr()), C.c_void_p(out.data_ptr()), x.numel(),
                                       C.c_void_p(_stream(x.device, stream))))
    return out


def momentum_stage(group: MuonGroup, beta: float, nesterov: bool, stream=None) -> torch.Tensor:
    _check_groups([group])
    mt = torch.empty((group.count, group.rows, group.cols), dtype=torch.float32, device=group.device)
    s, keep = group.to_c()
    L.check(L.lib().ma_test_muon_momentum(C.byref(s), beta, int(nesterov), C.c_void_p(mt.data_ptr()),
                                          C.c_void_p(_stream(group.device, stream))))
    return mt


def update_stage(group: MuonGroup, u: torch.Tensor, c_lr: float, c_wd: float, cautious: bool, decay: bool,
                 stream=None) -> None:
    if not u.is_contiguous():
        raise ValueError("u must be contiguous")
    _check_cuda([u], _check_groups([group]), "update_stage")
    s, keep = group.to_c()
    L.check(L.lib().ma_test_muon_update(C.byref(s), C.c_void_p(u.data_ptr()), _dt(u), c_lr, c_wd,
                                        int(cautious), int(decay), C.c_void_p(_stream(group.device, stream))))


def newton_schulz(x0: torch.Tensor, coeffs, ns_steps: int, stream=None) -> torch.Tensor:
    """Newton-Schulz iteration alone on ``[count, m, n]`` (m <= n), dtype bf16 or fp32."""
    if x0.dim() == 2:
        x0 = x0.unsqueeze(0)
    x0 = x0.contiguous()
    _check_cuda([x0], x0.device, "newton_schulz")
    count, m, n = x0.shape
    prec = _dt(x0)
    tab = MuonHParams(ns_steps=ns_steps, coeffs=coeffs).table()
    arr = (C.c_float * max(1, len(tab)))(*tab)
    need = L.lib().ma_test_ns_workspace_size(m, n, count, prec)
    if need == 0 and count > 0:
        L.check(L.MA_ERR_INVALID_ARG)
    ws = torch.empty(max(1, need), dtype=torch.uint8, device=x0.device)
    u = torch.empty_like(x0)
    L.check(L.lib().ma_test_ns(m, n, count, prec, C.c_void_p(x0.data_ptr()), C.c_void_p(u.data_ptr()),
                               C.cast(arr, C.POINTER(C.c_float)), ns_steps, C.c_void_p(ws.data_ptr()),
                               ws.numel(), C.c_void_p(_stream(x0.device, stream))))
    return u
