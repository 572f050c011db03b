"""Non-finite detection in the Muon step (``check_finite``), after the
fast-fail rule of "Chapter 4: The MuonAdamW Optimizer", section "Fast-Fail
on NaN or Loss > 100".

NaN, Inf and an overflowing entry are planted in the gradients or momentum
of a few matrices of a ragged multi-group step. With ``check_finite``:

* exactly the planted matrices are flagged (``ma_muon_nonfinite``), and the
  call reports MA_ERR_NONFINITE;
* a flagged matrix keeps its weight bit for bit;
* every other matrix -- weight and momentum -- is bit-identical to a step of
  the same inputs without the planted values;
* a step without planted values flags nothing and matches a step without the
  check bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_util import f32r, need_gpu, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
KJ = (3.4445, -4.7750, 2.0315)

# (rows, cols, count): one-pass wide groups, a tall group, a ragged tile-path group
SHAPES = [(256, 1024, 3), (300, 100, 2), (37, 53, 3), (128, 512, 2)]
# (group, matrix, buffer, row, col, value)
PLANTS = [(0, 1, "G", 5, 7, float("nan")), (1, 0, "G", 3, 2, float("inf")), (2, 2, "M", 0, 0, float("-inf")),
          (3, 1, "G", 0, 0, 1e30)]   # 1e30 squared overflows binary32


def _inputs(seed=11):
    g = torch.Generator().manual_seed(seed)
    out = []
    for R, C, n in SHAPES:
        W = (torch.randn(n, R, C, generator=g) * 0.02).to(torch.bfloat16)
        G = (torch.randn(n, R, C, generator=g) * 1e-3).to(torch.bfloat16)
        Mo = (torch.randn(n, R, C, generator=g) * 3e-3).to(torch.bfloat16)
        out.append([W, G, Mo])
    return out


def _step(host, eq, check, stats=False):
    import adamw_optimizer_step_amd as M
    dev = [[t.to(DEV).contiguous() for t in grp] for grp in host]
    groups = [M.MuonGroup(*grp) for grp in dev]
    hp = M.MuonHParams(lr=f32r(0.02), momentum=f32r(0.95), weight_decay=f32r(0.01), ns_steps=5, coeffs=KJ,
                       cautious=True, equilibrate=eq, ns_precision="bf16", check_finite=check)
    st = torch.zeros(2 * sum(g.count for g in groups), dtype=torch.float32, device=DEV) if stats else None
    ws = M.muon_step(groups, hp, stats=st)
    torch.cuda.synchronize()
    flags = M.muon_nonfinite(groups, hp, ws) if check else None
    return dev, flags, (st.cpu() if stats else None)


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy()


@pytest.mark.parametrize("eq", ["pre", "off", "post"])
def test_planted_nonfinite_values_are_flagged_and_contained(eq):
    need_gpu()
    clean = _inputs()
    planted = [[t.clone() for t in grp] for grp in clean]
    for gi, k, buf, r, c, v in PLANTS:
        planted[gi]["WGM".index(buf)][k, r, c] = v
    say("finite: clean step", eq)
    ref, flags_ref, _ = _step(clean, eq, True)
    assert not any(flags_ref)
    say("finite: clean step without the check", eq)
    plain, _, _ = _step(clean, eq, False)
    for a, b in zip(ref, plain):
        assert np.array_equal(_bits(a[0]), _bits(b[0])) and np.array_equal(_bits(a[2]), _bits(b[2]))
    say("finite: planted step", eq)
    got, flags, _ = _step(planted, eq, True)
    offsets = np.cumsum([0] + [n for _, _, n in SHAPES])
    expect = [False] * int(offsets[-1])
    for gi, k, *_ in PLANTS:
        expect[offsets[gi] + k] = True
    assert flags == expect
    for gi, (W0, _, _) in enumerate(planted):
        for k in range(W0.shape[0]):
            w = _bits(got[gi][0][k])
            if expect[offsets[gi] + k]:
                assert np.array_equal(w, _bits(W0[k])), f"group {gi} matrix {k}: flagged weight changed"
            else:
                assert np.array_equal(w, _bits(ref[gi][0][k])), f"group {gi} matrix {k}: weight differs"
                assert np.array_equal(_bits(got[gi][2][k]), _bits(ref[gi][2][k])), \
                    f"group {gi} matrix {k}: momentum differs"


def test_flagged_matrix_step_size_report():
    """With the step-size report, a flagged matrix reports a zero step and the
    norm of its (unchanged) weight; the others report what a clean step does."""
    need_gpu()
    clean = _inputs(12)
    planted = [[t.clone() for t in grp] for grp in clean]
    planted[0][1][2, 0, 0] = float("nan")
    say("finite: stats, clean")
    _, _, st_ref = _step(clean, "pre", True, stats=True)
    say("finite: stats, planted")
    _, flags, st = _step(planted, "pre", True, stats=True)
    assert flags[2] and sum(flags) == 1
    assert float(st[4]) == 0.0 and float(st[5]) == float(st_ref[5])
    keep = [i for i in range(len(flags)) if i != 2]
    for i in keep:
        assert float(st[2 * i]) == float(st_ref[2 * i]) and float(st[2 * i + 1]) == float(st_ref[2 * i + 1])
