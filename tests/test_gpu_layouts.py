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

The one-pass MuonEq PRE form (X0 stored before its Frobenius factor, which the
first Gram product and update apply) changes rounding, so it is compared with
the two-pass form to the bf16 iteration's tolerance instead.
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

# (rows, cols, count): wide, tall, and a padded odd shape of each orientation;
# 108 Gram jobs of 256 x 256, enough for the LDS-DMA kernel on every product
# (a launch of fewer than 64 runs its Gram and POLY on the register-staged
# kernel, which writes B with its mirrors)
SHAPES = [(512, 1280, 12), (1280, 512, 12), (300, 700, 6), (700, 300, 6)]

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
    # X0 from the separate passes in both runs: the one-pass form rounds X0
    # before its Frobenius factor, and it needs the transposed AXPY operands
    env["MA_PRE_ROWS"] = "0"
    here = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    assert here.returncode == 0, here.stderr[-2000:]
    say("layouts: both layouts of X and of B, in a child process")
    env.update(MA_NS_QT="0", MA_NS_SYMUP="0")
    both = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    assert both.returncode == 0, both.stderr[-2000:]
    a, b = _hashes(here.stdout), _hashes(both.stdout)
    assert set(a) == {0, 5} and a == b, (a, b)


ROWPASS_CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, {root!r})
import adamw_optimizer_step_amd as M
SHAPES = {shapes!r}
gen = torch.Generator().manual_seed(11)
groups, tensors = [], []
for r, c, n in SHAPES:
    W = (torch.randn(n, r, c, generator=gen) * 0.02).to(torch.bfloat16).cuda()
    G = (torch.randn(n, r, c, generator=gen) * 1e-3).to(torch.bfloat16).cuda()
    Mo = (torch.randn(n, r, c, generator=gen) * 3e-3).to(torch.bfloat16).cuda()
    groups.append(M.MuonGroup(W, G, Mo))
    tensors.append((W, Mo))
hp = M.MuonHParams(lr=0.02, momentum=0.95, weight_decay=0.01, ns_steps=5, coeffs=M.POLAR_EXPRESS,
                   cautious=True, equilibrate="pre", ns_precision="bf16")
print("rowpass", *[int(M.muon_row_pass(groups, hp, i)) for i in range(len(groups))], flush=True)
ws = M.muon_step(groups, hp)
torch.cuda.synchronize()
out = {{}}
for gi, (W, Mo) in enumerate(tensors):
    out[f"m{{gi}}"] = Mo.view(torch.int16).cpu().numpy()
    for k in range(W.shape[0]):
        out[f"u{{gi}}_{{k}}"] = M.muon_workspace_update(groups, hp, ws, gi, k).float().cpu().numpy()
np.savez({path!r}, **out)
"""

# (rows, cols, count): wide, square, and a padded one (300 -> 512 rows, 704 -> 768 columns)
ROWPASS_SHAPES = [(512, 1280, 3), (1024, 1024, 2), (300, 704, 2)]


def test_one_pass_x0_matches_two_passes(tmp_path):
    """MuonEq PRE in one pass over G and M (the Frobenius factor applied by
    the first Gram product and update) against the separate row-sum and X0
    passes (MA_PRE_ROWS=0): the stored momentum is bit-identical, the
    Newton-Schulz results agree to the bf16 iteration's tolerance."""
    import numpy as np
    need_gpu()
    res = {}
    for mode in ("one", "two"):
        path = str(tmp_path / f"{mode}.npz")
        env = dict(os.environ)
        env.pop("MA_NS_QT", None)
        env.pop("MA_NS_SYMUP", None)
        if mode == "two":
            env["MA_PRE_ROWS"] = "0"
        else:
            env.pop("MA_PRE_ROWS", None)
        say(f"row pass: {mode} pass(es), child process")
        code = ROWPASS_CHILD.format(root=ROOT, shapes=ROWPASS_SHAPES, path=path)
        p = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
        assert p.returncode == 0, p.stderr[-2000:]
        flags = [ln.split()[1:] for ln in p.stdout.splitlines() if ln.startswith("rowpass")][0]
        assert flags == (["1"] * 3 if mode == "one" else ["0"] * 3), flags
        res[mode] = dict(np.load(path))
    a, b = res["one"], res["two"]
    assert set(a) == set(b)
    for key in a:
        if key.startswith("m"):
            assert np.array_equal(a[key], b[key]), key
        else:
            x, y = a[key].astype(np.float64), b[key].astype(np.float64)
            err = np.linalg.norm(x - y) / np.linalg.norm(y)
            assert err <= 2e-2, (key, err)
