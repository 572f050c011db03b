"""ma_muon_step_noalloc against ma_muon_step: the same step with the
library's fixed per-GPU scratch array in place of a caller workspace gives
the same bits. Two calls in a row, the second with smaller matrices (and
other shapes), so that whatever the first call left in the shared array
must not leak into the second; then a third call that repeats the first.
"""
import numpy as np
import pytest
import torch

from gpu_util import f32r, need_gpu, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

CALLS = [
    # (shapes, MuonEq, ns_precision)
    ([(256, 256, 4), (1024, 256, 2), (256, 1024, 2)], "pre", "bf16"),
    ([(100, 300, 1), (37, 53, 2), (130, 66, 1)], "post", "bf16"),
    ([(256, 256, 4), (1024, 256, 2), (256, 1024, 2)], "pre", "bf16"),
    ([(64, 96, 2), (200, 40, 1)], "off", "f32"),
]


def _inputs(shapes, seed):
    g = torch.Generator().manual_seed(seed)
    return [[(torch.randn(n, r, c, generator=g) * s).to(torch.bfloat16) for s in (0.02, 1e-3, 3e-3)]
            for r, c, n in shapes]


def _bits(t):
    return t.cpu().view(torch.int16).numpy()


@pytest.mark.parametrize("_", [0])
def test_noalloc_step_matches_workspace_step(_):
    need_gpu()
    import adamw_optimizer_step_amd as M
    from adamw_optimizer_step_amd import _lib as L
    for i, (shapes, eq, prec) in enumerate(CALLS):
        host = _inputs(shapes, 40 + i)
        a = [[t.to(DEV) for t in grp] for grp in host]
        b = [[t.to(DEV) for t in grp] for grp in host]
        hp = M.MuonHParams(lr=f32r(0.02), momentum=f32r(0.95), weight_decay=f32r(0.01), ns_steps=5,
                           coeffs=M.KELLER_JORDAN, cautious=True, equilibrate=eq, ns_precision=prec)
        ga = [M.MuonGroup(*grp) for grp in a]
        gb = [M.MuonGroup(*grp) for grp in b]
        assert M.muon_workspace_size(ga, hp) <= L.MA_NOALLOC_SCRATCH_BYTES
        say("noalloc call", i, shapes, eq, prec)
        M.muon_step(ga, hp)
        M.muon_step_noalloc(gb, hp)
        torch.cuda.synchronize()
        for gi, (x, y) in enumerate(zip(a, b)):
            assert np.array_equal(_bits(x[0]), _bits(y[0])), f"call {i} group {gi}: weights differ"
            assert np.array_equal(_bits(x[2]), _bits(y[2])), f"call {i} group {gi}: momentum differs"
