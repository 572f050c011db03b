"""The bf16 iteration's layout choices leave every result bit-identical.

By default AXPY reads X^T out of the row-major X through transposing LDS reads
(so no X^T copy is written), and POLY writes each symmetric tile of B once,
AXPY reading the blocks left of the diagonal transposed from those above it.
With MA_NS_QT=0 and MA_NS_SYMUP=0 the library keeps both layouts of X and
both triangles of B instead. Both forms multiply the same values in the same
order, so a seeded Muon step must give the same bits either way: this test
runs the step in two child processes (the switches are read once per
process), with the defaults and with both switches off, for wide, tall and
padded bf16 matrices, with five steps and with none.
"""
import hashlib
import os
import subprocess
import sys

import pytest
import torch

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (rows, cols, count): wide, tall, and a padded odd shape of each orientation
SHAPES = [(512, 1280, 3), (1280, 512, 3), (300, 700, 2), (700, 300, 2)]

CHILD = r"""
import hashlib, sys, torch
sys.path.insert(0, {root!r})
import adamw_optimizer_step_amd as M
SHAPES = {shapes!r}
for ns_steps in (5, 0):
    gen = torch.Generator().manual_seed(5 + ns_steps)
    groups, tensors = [], []
    for r, c, n in SHAPES:
        W = (torch.randn(n, r, c, generator=gen) * 0.02).to(torch.bfloat16).cuda()
        G = (torch.randn(n, r, c, generator=gen) * 1e-3).to(torch.bfloat16).cuda()
        Mo = (torch.randn(n, r, c, generator=gen) * 3e-3).to(torch.bfloat16).cuda()
        groups.append(M.MuonGroup(W, G, Mo))
        tensors.append((W, Mo))
    coeffs = M.POLAR_EXPRESS if ns_steps == 5 else M.KELLER_JORDAN   # one triple per step, or one for all
    hp = M.MuonHParams(lr=0.02, momentum=0.95, weight_decay=0.01, ns_steps=ns_steps, coeffs=coeffs,
                       cautious=True, equilibrate="pre", ns_precision="bf16")
    M.muon_step(groups, hp)
    torch.cuda.synchronize()
    h = hashlib.sha256()
    for W, Mo in tensors:
        h.update(W.view(torch.int16).cpu().numpy().tobytes())
        h.update(Mo.view(torch.int16).cpu().numpy().tobytes())
    print("hash", ns_steps, h.hexdigest(), flush=True)
"""


def _hashes(out):
    return {int(p[1]): p[2] for p in (line.split() for line in out.splitlines()) if p and p[0] == "hash"}


def test_transposed_operands_are_bit_identical_to_both_layouts():
    need_gpu()
    code = CHILD.format(root=ROOT, shapes=SHAPES)
    say("layouts: default (X^T read from X, B stored once), child process")
    env = dict(os.environ)
    env.pop("MA_NS_QT", None)
    env.pop("MA_NS_SYMUP", None)
    here = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    assert here.returncode == 0, here.stderr[-2000:]
    say("layouts: both layouts of X and of B, in a child process")
    env.update(MA_NS_QT="0", MA_NS_SYMUP="0")
    both = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    assert both.returncode == 0, both.stderr[-2000:]
    a, b = _hashes(here.stdout), _hashes(both.stdout)
    assert set(a) == {0, 5} and a == b, (a, b)
