"""Checkpoint and resume. All optimizer state is caller-owned device memory
-- the weights, the Muon momentum buffers, AdamW's parameters and moments and
its step count -- and every kernel is deterministic, so k steps, a
checkpoint of that state, and k more steps from the checkpoint in fresh
buffers give the bits of 2k uninterrupted steps. The continuation is run
eagerly and as captured HIP graphs replayed (one graph per AdamW step count,
a host scalar baked into the capture).
"""
import io

import numpy as np
import pytest
import torch

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
K = 2


def _initial(seed=21):
    g = torch.Generator().manual_seed(seed)
    muon = []
    for r, c, n in [(256, 768, 3), (768, 256, 2), (100, 300, 2)]:
        muon.append({"W": (torch.randn(n, r, c, generator=g) * 0.02).to(torch.bfloat16),
                     "M": torch.zeros(n, r, c, dtype=torch.bfloat16)})
    ad = {"p": torch.randn(70001, generator=g) * 0.02, "m": torch.zeros(70001), "v": torch.zeros(70001)}
    grads = [[(torch.randn(grp["W"].shape, generator=g) * 1e-3).to(torch.bfloat16) for grp in muon]
             for _ in range(2 * K)]
    agrads = [torch.randn(70001, generator=g) * 1e-3 for _ in range(2 * K)]
    return {"muon": muon, "adamw": ad, "t": 0}, grads, agrads


def _to(state, device):
    return {"muon": [{k: v.to(device).contiguous() for k, v in grp.items()} for grp in state["muon"]],
            "adamw": {k: v.to(device).contiguous() for k, v in state["adamw"].items()}, "t": state["t"]}


class Runner:
    """One optimizer on device state; gradients are copied into its buffers."""

    def __init__(self, state):
        import adamw_optimizer_step_amd as M
        self.M = M
        self.s = _to(state, DEV)
        self.g = [torch.empty_like(grp["W"]) for grp in self.s["muon"]]
        self.ag = torch.empty_like(self.s["adamw"]["p"])
        self.groups = [M.MuonGroup(grp["W"], g, grp["M"]) for grp, g in zip(self.s["muon"], self.g)]
        self.hp = M.MuonHParams(lr=0.02, momentum=0.95, weight_decay=0.01, ns_steps=5, coeffs=M.KELLER_JORDAN,
                                cautious=True, equilibrate="pre", ns_precision="bf16")
        self.ws = torch.empty(max(1, M.muon_workspace_size(self.groups, self.hp)), dtype=torch.uint8, device=DEV)

    def segs(self, t):
        a = self.s["adamw"]
        return [dict(param=a["p"], grad=self.ag, exp_avg=a["m"], exp_avg_sq=a["v"], step=t, lr=3e-4,
                     beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)]

    def load_grads(self, gs, ag):
        for dst, src in zip(self.g, gs):
            dst.copy_(src.to(DEV))
        self.ag.copy_(ag.to(DEV))

    def step(self, gs, ag):
        self.load_grads(gs, ag)
        self.s["t"] += 1
        self.M.optimizer_step(self.groups, self.hp, self.segs(self.s["t"]), workspace=self.ws, overlap=True)

    def checkpoint(self):
        torch.cuda.synchronize()
        buf = io.BytesIO()
        torch.save(_to(self.s, "cpu"), buf)   # the caller's own checkpoint
        buf.seek(0)
        return torch.load(buf, weights_only=True)

    def bits(self):
        torch.cuda.synchronize()
        out = [t.cpu().view(torch.int16).numpy() for grp in self.s["muon"] for t in (grp["W"], grp["M"])]
        out += [self.s["adamw"][k].cpu().view(torch.int32).numpy() for k in ("p", "m", "v")]
        return out


def test_resume_from_checkpoint_is_bit_identical():
    need_gpu()
    init, grads, agrads = _initial()
    say("resume: uninterrupted run")
    a = Runner(init)
    for i in range(K):
        a.step(grads[i], agrads[i])
    ckpt = a.checkpoint()
    for i in range(K, 2 * K):
        a.step(grads[i], agrads[i])
    want = a.bits()

    say("resume: eager continuation from the checkpoint")
    b = Runner(ckpt)
    assert b.s["t"] == K
    for i in range(K, 2 * K):
        b.step(grads[i], agrads[i])
    for i, (x, y) in enumerate(zip(want, b.bits())):
        assert np.array_equal(x, y), f"eager resume: tensor {i} differs"

    say("resume: continuation as captured graphs")
    c = Runner(ckpt)
    graphs = []
    cap = torch.cuda.Stream(DEV)
    cap.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(cap):   # warm the capture stream on a scratch copy
        w = Runner(ckpt)
        w.step(grads[K], agrads[K])
    torch.cuda.current_stream(DEV).wait_stream(cap)
    torch.cuda.synchronize()
    for i in range(K, 2 * K):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            t = K + 1 + (i - K)
            c.M.optimizer_step(c.groups, c.hp, c.segs(t), workspace=c.ws, overlap=True)
        graphs.append(g)
    for i, g in zip(range(K, 2 * K), graphs):
        c.load_grads(grads[i], agrads[i])
        g.replay()
        junk = torch.randn(1 << 16, device=DEV).sum()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
    for i, (x, y) in enumerate(zip(want, c.bits())):
        assert np.array_equal(x, y), f"graph resume: tensor {i} differs"
