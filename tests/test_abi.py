"""The C ABI without a GPU: the library loads, exports every entry point that
include/muon_adamw.h declares, and rejects bad arguments before any launch
(so these calls never reach the HIP runtime)."""
import ctypes as C
import os
import re

import pytest

from adamw_optimizer_step_amd import _lib as L
from adamw_optimizer_step_amd.api import MuonHParams

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon_adamw.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ma_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol():
    h = C.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(h, name), name


def test_library_links_roctx():
    """The entry points mark their host-side work as roctx ranges, so the
    library needs the roctx runtime (a no-op unless a profiler is attached)."""
    import subprocess
    out = subprocess.run(["readelf", "-d", L.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert re.search(r"NEEDED.*librocprofiler-sdk-roctx", out), out


def test_status_strings_and_version():
    lib = L.lib()
    assert lib.ma_status_string(0) == b"ok"
    for code in (L.MA_ERR_INVALID_ARG, L.MA_ERR_UNSUPPORTED, L.MA_ERR_WORKSPACE, L.MA_ERR_HIP):
        assert lib.ma_status_string(code) not in (b"ok", b"unknown status")
    assert b"gfx950" in lib.ma_version()


# fake, never dereferenced device addresses (validation fails before any launch)
BASE = 1 << 40


def group(rows=64, cols=128, count=2, dts=(1, 1, 1), base=BASE, gap=1 << 24):
    p = (C.c_void_p * count)(*[base + 3 * i * gap for i in range(count)])
    g = (C.c_void_p * count)(*[base + (3 * i + 1) * gap for i in range(count)])
    m = (C.c_void_p * count)(*[base + (3 * i + 2) * gap for i in range(count)])
    s = L.MuonGroupC(rows=rows, cols=cols, count=count, param_dtype=dts[0], grad_dtype=dts[1],
                     mom_dtype=dts[2], params=C.cast(p, C.POINTER(C.c_void_p)),
                     grads=C.cast(g, C.POINTER(C.c_void_p)), momentum=C.cast(m, C.POINTER(C.c_void_p)))
    return s, (p, g, m)


def hp(**kw):
    h, tab = MuonHParams(**kw).to_c()
    return h, tab


def call_step(g, h, ws=BASE * 4, nbytes=1 << 40):
    arr = (L.MuonGroupC * 1)(g)
    return L.lib().ma_muon_step(arr, 1, C.byref(h), C.c_void_p(ws), nbytes, None)


def test_workspace_size_lower_bound():
    g, k = group(rows=1024, cols=4096, count=3)
    h, t = hp()
    n = L.lib().ma_muon_workspace_size((L.MuonGroupC * 1)(g), 1, C.byref(h))
    # bf16: X (two buffers) plus two m x m Gram buffers; X^T is read out of X
    assert n >= 3 * (2 * 1024 * 4096 + 2 * 1024 * 1024) * 2
    g2, k2 = group(rows=4096, cols=1024, count=3)   # tall: X^T also holds the parameter's layout
    n2 = L.lib().ma_muon_workspace_size((L.MuonGroupC * 1)(g2), 1, C.byref(h))
    assert n2 >= n + 3 * 2 * 1024 * 4096 * 2
    h32, t32 = hp(ns_precision="f32")   # fp32: X and X^T, 4-byte elements
    assert L.lib().ma_muon_workspace_size((L.MuonGroupC * 1)(g), 1, C.byref(h32)) >= 2 * n2 - (1 << 20)


@pytest.mark.parametrize("rows,cols,kw,base,expect", [
    (1024, 1024, {}, BASE, 1),
    (1024, 4096, {}, BASE, 1),
    (20, 1000, {}, BASE, 1),                       # 1000 columns pad to 1024
    (4096, 1024, {}, BASE, 0),                     # tall: the iteration runs on X^T
    (1024, 4104, {}, BASE, 0),                     # 4104 pads to 4352 > 4096
    (100, 300, {}, BASE, 0),                       # cols % 8 != 0: no vector path
    (1024, 1024, {}, BASE + 8, 0),                 # 8-byte aligned buffers
    (1024, 1024, dict(equilibrate="off"), BASE, 0),
    (1024, 1024, dict(equilibrate="post"), BASE, 0),
    (1024, 1024, dict(ns_steps=0), BASE, 0),
    (1024, 1024, dict(ns_precision="f32"), BASE, 0),
])
def test_row_pass_predicate(rows, cols, kw, base, expect):
    """Which groups ma_muon_step reads in one pass (host-only query)."""
    if os.environ.get("MA_PRE_ROWS") == "0" or os.environ.get("MA_NS_QT") == "0":
        pytest.skip("one-pass form switched off in this environment")
    g, k = group(rows=rows, cols=cols, count=2, base=base)
    args = dict(equilibrate="pre", ns_steps=5)
    args.update(kw)
    h, t = hp(**args)
    assert L.lib().ma_muon_row_pass((L.MuonGroupC * 1)(g), 1, C.byref(h), 0) == expect
    assert L.lib().ma_muon_row_pass((L.MuonGroupC * 1)(g), 1, C.byref(h), 1) == L.MA_ERR_INVALID_ARG


@pytest.mark.parametrize("mut,code", [
    (lambda g, h: setattr(h, "ns_steps", 17), L.MA_ERR_INVALID_ARG),
    (lambda g, h: setattr(h, "ns_steps", -1), L.MA_ERR_INVALID_ARG),
    (lambda g, h: setattr(h, "abc", None), L.MA_ERR_INVALID_ARG),
    (lambda g, h: setattr(h, "equilibrate", 7), L.MA_ERR_INVALID_ARG),
    (lambda g, h: setattr(h, "lr_scale", 5), L.MA_ERR_INVALID_ARG),
    (lambda g, h: setattr(h, "ns_precision", 3), L.MA_ERR_UNSUPPORTED),
    (lambda g, h: setattr(h, "lr", float("nan")), L.MA_ERR_INVALID_ARG),
    (lambda g, h: setattr(g, "rows", 0), L.MA_ERR_INVALID_ARG),
    (lambda g, h: setattr(g, "cols", -4), L.MA_ERR_INVALID_ARG),
    (lambda g, h: setattr(g, "param_dtype", 9), L.MA_ERR_UNSUPPORTED),
    (lambda g, h: setattr(g, "params", None), L.MA_ERR_INVALID_ARG),
])
def test_muon_step_rejects_bad_arguments(mut, code):
    g, keep = group()
    h, tab = hp()
    mut(g, h)
    assert call_step(g, h) == code
    assert L.lib().ma_last_error()


def test_muon_step_rejects_groups_beyond_the_size_bound():
    # 1025 matrices of 2^15 x 2^15: each allowed, more than 2^40 elements in all
    g, keep = group(rows=1 << 15, cols=1 << 15, count=1025)
    h, tab = hp()
    assert call_step(g, h) == L.MA_ERR_INVALID_ARG
    assert b"2^40" in L.lib().ma_last_error()
    assert L.lib().ma_muon_workspace_size((L.MuonGroupC * 1)(g), 1, C.byref(h)) == 0


def test_muon_step_rejects_null_matrix_pointer():
    g, (p, gg, m) = group()
    gg[1] = None
    h, tab = hp()
    assert call_step(g, h) == L.MA_ERR_INVALID_ARG


def test_muon_step_rejects_misaligned_pointer():
    g, (p, gg, m) = group()
    p[0] = BASE + 1          # bf16 needs 2-byte alignment
    h, tab = hp()
    assert call_step(g, h) == L.MA_ERR_INVALID_ARG


def test_muon_step_workspace_checks():
    g, keep = group()
    h, tab = hp()
    assert call_step(g, h, ws=0) == L.MA_ERR_WORKSPACE
    assert call_step(g, h, ws=BASE * 4 + 8) == L.MA_ERR_WORKSPACE
    assert call_step(g, h, nbytes=1024) == L.MA_ERR_WORKSPACE


def test_muon_step_rejects_overlaps():
    g, (p, gg, m) = group(rows=64, cols=128)
    gg[0] = p[0] + 64          # gradient overlaps a weight
    h, tab = hp()
    assert call_step(g, h) == L.MA_ERR_INVALID_ARG
    g, (p, gg, m) = group()
    h, tab = hp()
    assert call_step(g, h, ws=p[1] - 256) == L.MA_ERR_INVALID_ARG   # workspace over a weight


def test_muon_step_stats_validates_stats_pointer():
    g, (p, gg, m) = group(rows=64, cols=128)
    h, tab = hp()
    arr = (L.MuonGroupC * 1)(g)
    lib = L.lib()
    call = lambda st: lib.ma_muon_step_stats(arr, 1, C.byref(h), C.c_void_p(BASE * 4), 1 << 40, st, None)
    assert call(None) == L.MA_ERR_INVALID_ARG                          # null
    assert call(C.c_void_p(BASE * 8 + 2)) == L.MA_ERR_INVALID_ARG      # not 4-byte aligned
    assert call(C.c_void_p(p[0] + 64)) == L.MA_ERR_INVALID_ARG         # overlaps a weight
    assert call(C.c_void_p(BASE * 4 + 512)) == L.MA_ERR_INVALID_ARG    # inside the workspace


def seg(**kw):
    d = dict(param=BASE, grad=BASE + (1 << 30), exp_avg=BASE + (2 << 30), exp_avg_sq=BASE + (3 << 30),
             n=1000, param_dtype=0, grad_dtype=0, lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8,
             weight_decay=0.0, step=1)
    d.update(kw)
    return L.AdamWSegmentC(**d)


@pytest.mark.parametrize("kw,code", [
    (dict(step=0), L.MA_ERR_INVALID_ARG),
    (dict(n=-1), L.MA_ERR_INVALID_ARG),
    (dict(param_dtype=1), L.MA_ERR_UNSUPPORTED),
    (dict(beta1=1.0), L.MA_ERR_INVALID_ARG),
    (dict(beta2=-0.1), L.MA_ERR_INVALID_ARG),
    (dict(lr=float("inf")), L.MA_ERR_INVALID_ARG),
    (dict(grad=None), L.MA_ERR_INVALID_ARG),
    (dict(param=BASE + 2), L.MA_ERR_INVALID_ARG),
    (dict(exp_avg=BASE + 400), L.MA_ERR_INVALID_ARG),     # overlaps param
    (dict(n=(1 << 40) + 1), L.MA_ERR_INVALID_ARG),        # beyond the size bound
])
def test_adamw_rejects_bad_arguments(kw, code):
    arr = (L.AdamWSegmentC * 1)(seg(**kw))
    assert L.lib().ma_adamw_step(arr, 1, None) == code


def test_adamw_background_validates_workgroups():
    seg = L.AdamWSegmentC(param=BASE, grad=BASE + (1 << 24), exp_avg=BASE + (2 << 24), exp_avg_sq=BASE + (3 << 24),
                          n=1000, param_dtype=0, grad_dtype=0, lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                          weight_decay=0.0, step=1)
    arr = (L.AdamWSegmentC * 1)(seg)
    for wg in (0, -1):
        assert L.lib().ma_adamw_step_background(arr, 1, wg, None) == L.MA_ERR_INVALID_ARG
    assert L.lib().ma_adamw_step_background(None, 0, 256, None) == 0


def test_muon_adamw_step_validates_before_launch():
    g, k = group(rows=64, cols=128, count=2)
    h, t = hp()
    garr = (L.MuonGroupC * 1)(g)
    seg = L.AdamWSegmentC(param=BASE * 2, grad=BASE * 2 + (1 << 24), exp_avg=BASE * 2 + (2 << 24),
                          exp_avg_sq=BASE * 2 + (3 << 24), n=1000, param_dtype=0, grad_dtype=0, lr=1e-3,
                          beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, step=1)
    arr = (L.AdamWSegmentC * 1)(seg)
    lib = L.lib()
    ws, nb = C.c_void_p(BASE * 4), 1 << 40
    s1, s2 = C.c_void_p(0x1000), C.c_void_p(0x2000)
    assert lib.ma_muon_adamw_step(garr, 1, C.byref(h), ws, nb, arr, 1, 0, s1, s2) == L.MA_ERR_INVALID_ARG
    assert lib.ma_muon_adamw_step(garr, 1, C.byref(h), ws, nb, arr, 1, 256, s1, s1) == L.MA_ERR_INVALID_ARG
    bad = L.AdamWSegmentC(param=BASE * 2, grad=BASE * 2, exp_avg=BASE * 2 + (2 << 24),   # grad aliases param
                          exp_avg_sq=BASE * 2 + (3 << 24), n=1000, param_dtype=0, grad_dtype=0, lr=1e-3,
                          beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, step=1)
    assert lib.ma_muon_adamw_step(garr, 1, C.byref(h), ws, nb, (L.AdamWSegmentC * 1)(bad), 1, 256, s1,
                                  s2) == L.MA_ERR_INVALID_ARG


def test_muon_adamw_step_rejects_overlap_between_the_two_steps():
    """AdamW runs concurrently with the Muon step, so an AdamW buffer over a
    Muon buffer or the workspace is rejected before anything is enqueued."""
    g, (p, gg, m) = group(rows=64, cols=128, count=2)
    h, t = hp()
    garr = (L.MuonGroupC * 1)(g)
    lib = L.lib()
    ws, nb = BASE * 4, 1 << 40
    s1, s2 = C.c_void_p(0x1000), C.c_void_p(0x2000)
    call = lambda sg: lib.ma_muon_adamw_step(garr, 1, C.byref(h), C.c_void_p(ws), nb,
                                             (L.AdamWSegmentC * 1)(sg), 1, 256, s1, s2)
    far = BASE * 2
    ok = dict(param=far, grad=far + (1 << 24), exp_avg=far + (2 << 24), exp_avg_sq=far + (3 << 24))
    # exp_avg over a Muon weight
    assert call(seg(**{**ok, "exp_avg": p[1] + 128})) == L.MA_ERR_INVALID_ARG
    assert "overlap" in lib.ma_last_error().decode()
    # exp_avg_sq inside the workspace
    assert call(seg(**{**ok, "exp_avg_sq": ws + 4096})) == L.MA_ERR_INVALID_ARG
    # AdamW param over a Muon momentum buffer
    assert call(seg(**{**ok, "param": m[0]})) == L.MA_ERR_INVALID_ARG


def test_noalloc_step_rejects_steps_beyond_its_scratch():
    lib = L.lib()
    h, t = hp()
    small, k1 = group(rows=256, cols=1024, count=2)
    need = lib.ma_muon_workspace_size((L.MuonGroupC * 1)(small), 1, C.byref(h))
    assert 0 < need <= L.MA_NOALLOC_SCRATCH_BYTES
    big, k2 = group(rows=1024, cols=4096, count=8)
    assert lib.ma_muon_workspace_size((L.MuonGroupC * 1)(big), 1, C.byref(h)) > L.MA_NOALLOC_SCRATCH_BYTES
    assert lib.ma_muon_step_noalloc((L.MuonGroupC * 1)(big), 1, C.byref(h), None) == L.MA_ERR_WORKSPACE
    assert b"scratch" in lib.ma_last_error()
    g, (p, gg, m) = group(rows=64, cols=128)
    gg[0] = p[0] + 64          # the usual argument checks come first
    assert lib.ma_muon_step_noalloc((L.MuonGroupC * 1)(g), 1, C.byref(h), None) == L.MA_ERR_INVALID_ARG


def test_check_finite_field_and_query_validate():
    g, k = group()
    h, t = hp()
    h.check_finite = 2
    assert call_step(g, h) == L.MA_ERR_INVALID_ARG
    lib = L.lib()
    arr = (L.MuonGroupC * 1)(g)
    flags = (C.c_int32 * 2)()
    h0, t0 = hp()   # check_finite off: the step wrote no flags, so there is nothing to read
    assert lib.ma_muon_nonfinite(arr, 1, C.byref(h0), C.c_void_p(BASE * 4), flags) == L.MA_ERR_INVALID_ARG
    h1, t1 = hp(check_finite=True)
    assert lib.ma_muon_nonfinite(arr, 1, C.byref(h1), None, flags) == L.MA_ERR_WORKSPACE
    assert lib.ma_status_string(L.MA_ERR_NONFINITE) not in (b"ok", b"unknown status")
    assert h1.check_finite == 1


def test_launching_calls_reject_host_tensors():
    """The binding refuses, before any library call, tensors that are not on
    the GPU: the kernels would get host addresses."""
    import torch
    from adamw_optimizer_step_amd import api
    W = torch.zeros(2, 8, 16, dtype=torch.bfloat16)
    grp = api.MuonGroup(W, torch.zeros_like(W), torch.zeros_like(W))
    hp = api.MuonHParams(ns_steps=1)
    for call in (lambda: api.muon_step([grp], hp), lambda: api.muon_step_noalloc([grp], hp),
                 lambda: api.momentum_stage(grp, 0.9, True), lambda: api.newton_schulz(W[0].float(), api.KELLER_JORDAN, 1),
                 lambda: api.bf16_round(torch.zeros(4))):
        with pytest.raises(ValueError, match="CUDA"):
            call()
    p = torch.zeros(8)
    seg = dict(param=p, grad=torch.zeros(8), exp_avg=torch.zeros(8), exp_avg_sq=torch.zeros(8), lr=1e-3, step=1)
    with pytest.raises(ValueError, match="CUDA"):
        api.adamw_step([seg])
    with pytest.raises(ValueError, match="CUDA"):
        api.lion_step([dict(param=p, grad=torch.zeros(8), exp_avg=torch.zeros(8), lr=1e-3)])
    with pytest.raises(ValueError, match="CUDA"):
        api.optimizer_step([grp], hp, [seg])


def test_missing_gradients_are_left_out_and_sparse_ones_rejected():
    """The wrapper drops matrices and AdamW buffers whose gradient is None
    (CPU tensors: only pointers are taken, nothing is launched)."""
    import torch
    from adamw_optimizer_step_amd import api
    W = torch.zeros(3, 8, 16, dtype=torch.bfloat16)
    Mo = torch.zeros_like(W)
    G = [torch.zeros(8, 16, dtype=torch.bfloat16), None, torch.zeros(8, 16, dtype=torch.bfloat16)]
    grp = api.MuonGroup(W, G, Mo)
    assert grp.count == 2 and grp.kept == [0, 2]
    step = 8 * 16 * 2
    assert grp.p == [W.data_ptr(), W.data_ptr() + 2 * step] and grp.m == [Mo.data_ptr(), Mo.data_ptr() + 2 * step]
    assert api.MuonGroup(W, None, Mo).count == 0
    assert api.MuonGroup(W, torch.zeros_like(W), Mo).count == 3
    sparse = torch.zeros(8, 16).to_sparse()
    with pytest.raises(TypeError):
        api.MuonGroup([W[0]], [sparse], [Mo[0]])
    p = torch.zeros(10)
    segs = [dict(param=p, grad=None, exp_avg=p, exp_avg_sq=p, lr=1.0, step=1),
            dict(param=torch.zeros(4), grad=torch.zeros(4), exp_avg=torch.zeros(4), exp_avg_sq=torch.zeros(4),
                 lr=1.0, step=1)]
    arr, n = api._adamw_c(segs)
    assert n == 1 and arr[0].n == 4
    with pytest.raises(TypeError):
        api._adamw_c([dict(param=p, grad=torch.zeros(10).to_sparse(), exp_avg=p, exp_avg_sq=p, lr=1.0, step=1)])


def test_adamw_zero_segments_is_noop():
    assert L.lib().ma_adamw_step(None, 0, None) == L.MA_OK
    arr = (L.AdamWSegmentC * 1)(seg(n=0, param=None, grad=None, exp_avg=None, exp_avg_sq=None))
    assert L.lib().ma_adamw_step(arr, 1, None) == L.MA_OK


def lseg(**kw):
    d = dict(param=BASE, grad=BASE + (1 << 30), exp_avg=BASE + (2 << 30), n=1000, param_dtype=0,
             grad_dtype=0, lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.0)
    d.update(kw)
    return L.LionSegmentC(**d)


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), L.MA_ERR_INVALID_ARG),
    (dict(param_dtype=1), L.MA_ERR_UNSUPPORTED),
    (dict(grad_dtype=1), L.MA_ERR_UNSUPPORTED),
    (dict(beta1=1.0), L.MA_ERR_INVALID_ARG),
    (dict(beta2=-0.1), L.MA_ERR_INVALID_ARG),
    (dict(beta1=float("nan")), L.MA_ERR_INVALID_ARG),
    (dict(lr=float("inf")), L.MA_ERR_INVALID_ARG),
    (dict(weight_decay=float("nan")), L.MA_ERR_INVALID_ARG),
    (dict(exp_avg=None), L.MA_ERR_INVALID_ARG),
    (dict(grad=BASE + (1 << 30) + 2), L.MA_ERR_INVALID_ARG),
    (dict(grad=BASE + 3996), L.MA_ERR_INVALID_ARG),          # overlaps param's last element
    (dict(n=(1 << 40) + 1), L.MA_ERR_INVALID_ARG),           # beyond the size bound
])
def test_lion_rejects_bad_arguments(kw, code):
    arr = (L.LionSegmentC * 1)(lseg(**kw))
    assert L.lib().ma_lion_step(arr, 1, None) == code


def test_lion_zero_segments_is_noop():
    assert L.lib().ma_lion_step(None, 0, None) == L.MA_OK
    assert L.lib().ma_lion_step(None, -1, None) == L.MA_ERR_INVALID_ARG
    arr = (L.LionSegmentC * 1)(lseg(n=0, param=None, grad=None, exp_avg=None))
    assert L.lib().ma_lion_step(arr, 1, None) == L.MA_OK


def test_stage_entry_points_validate():
    lib = L.lib()
    assert lib.ma_test_bf16_round(None, None, 10, None) == L.MA_ERR_INVALID_ARG
    assert lib.ma_test_ns_workspace_size(8, 4, 1, 1) == 0           # m > n
    assert lib.ma_test_ns(8, 4, 1, 1, None, None, None, 0, None, 0, None) == L.MA_ERR_INVALID_ARG
    g, keep = group()
    assert lib.ma_test_muon_update(C.byref(g), None, 1, 0.1, 0.0, 1, 1, None) == L.MA_ERR_INVALID_ARG


def test_hparams_table():
    assert MuonHParams(ns_steps=2).table() == pytest.approx([3.4445, -4.775, 2.0315] * 2)
    with pytest.raises(ValueError):
        MuonHParams(ns_steps=2, coeffs=[(1, 0, 0)] * 3).table()
    assert MuonHParams(ns_steps=2, coeffs=[(1, 0, 0), (2, 0, 0)]).table() == [1, 0, 0, 2, 0, 0]


def test_calib_mfma_validates():
    lib = L.lib()
    assert lib.ma_calib_mfma(0, 10, 0, C.c_void_p(BASE), None) == L.MA_ERR_INVALID_ARG
    assert lib.ma_calib_mfma(4, 0, 0, C.c_void_p(BASE), None) == L.MA_ERR_INVALID_ARG
    assert lib.ma_calib_mfma(4, 10, 0, None, None) == L.MA_ERR_INVALID_ARG
    assert lib.ma_calib_mfma(4, 10, 2, C.c_void_p(BASE), None) == L.MA_ERR_INVALID_ARG
    assert lib.ma_calib_mfma(4, 10, 0, C.c_void_p(BASE + 2), None) == L.MA_ERR_INVALID_ARG
