"""A Muon + AdamW step captured in a HIP graph and replayed gives, replay by
replay, the same bits as the same step launched eagerly.

The library launches only kernels on the caller's stream (no allocation, no
memset, no host synchronisation), so a whole optimizer step can be captured.
Each replay is checked against an eager step from the same state, with the
program's own eager work and synchronisations between replays. The captured
step runs AdamW either after the Muon step or on a second stream beside it
(forked and joined inside the capture); the eager reference runs them in turn.
"""
import numpy as np
import pytest
import torch

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _state(seed):
    g = torch.Generator().manual_seed(seed)
    shapes = [(256, 256, 3), (512, 256, 2), (256, 768, 2)]
    muon = []
    for r, c, n in shapes:
        W = (torch.randn(n, r, c, generator=g) * 0.02).to(torch.bfloat16)
        G = (torch.randn(n, r, c, generator=g) * 1e-3).to(torch.bfloat16)
        M = (torch.randn(n, r, c, generator=g) * 3e-3).to(torch.bfloat16)
        muon.append([W, G, M])
    ad = [torch.randn(100003, generator=g) * 0.02, torch.randn(100003, generator=g) * 1e-3,
          torch.randn(100003, generator=g) * 3e-4, torch.randn(100003, generator=g).square() * 1e-6]
    return muon, ad


def _to_dev(muon, ad):
    return [[t.to(DEV).contiguous() for t in grp] for grp in muon], [t.to(DEV).contiguous() for t in ad]


def _stepper(M, muon, ad, ws, overlap=False):
    groups = [M.MuonGroup(W, G, Mo) for W, G, Mo in muon]
    hp = M.MuonHParams(lr=0.02, momentum=0.95, weight_decay=0.01, nesterov=True, ns_steps=5,
                       coeffs=M.KELLER_JORDAN, cautious=True, equilibrate="pre", ns_precision="bf16")
    seg = [dict(param=ad[0], grad=ad[1], exp_avg=ad[2], exp_avg_sq=ad[3], step=7, lr=3e-4, beta1=0.9,
                beta2=0.95, eps=1e-8, weight_decay=0.1)]

    def step():
        if overlap:
            # AdamW forked onto a second stream and joined: two branches in the graph
            M.optimizer_step(groups, hp, seg, workspace=ws, overlap=True)
        else:
            M.muon_step(groups, hp, workspace=ws)
            M.adamw_step(seg)
    return groups, hp, step


def _snapshot(muon, ad):
    return [t.detach().cpu().view(torch.int16).numpy().copy() for grp in muon for t in (grp[0], grp[2])] + \
           [t.detach().cpu().view(torch.int32).numpy().copy() for t in (ad[0], ad[2], ad[3])]


@pytest.mark.parametrize("overlap", [False, True])
def test_graph_replays_match_eager_steps(overlap):
    need_gpu()
    import adamw_optimizer_step_amd as M
    init_m, init_a = _state(3)
    # eager reference
    em, ea = _to_dev(init_m, init_a)
    groups, hp, estep = _stepper(M, em, ea, None)
    ews = torch.empty(max(1, M.muon_workspace_size(groups, hp)), dtype=torch.uint8, device=DEV)
    groups, hp, estep = _stepper(M, em, ea, ews)
    # graph copy: warm up on the capture stream, reset the state, capture
    gm, ga = _to_dev(init_m, init_a)
    gws = torch.empty_like(ews)
    _, _, gstep = _stepper(M, gm, ga, gws, overlap=overlap)
    cap = torch.cuda.Stream(DEV)
    cap.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(cap):
        gstep()
    torch.cuda.current_stream(DEV).wait_stream(cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gstep()
    for dst, src in zip([t for grp in gm for t in grp] + ga, [t for grp in init_m for t in grp] + init_a):
        dst.copy_(src.to(DEV))
    torch.cuda.synchronize()
    for k in range(3):
        say("graph replay", k)
        estep()
        graph.replay()
        # unrelated eager work between replays
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        a, b = _snapshot(em, ea), _snapshot(gm, ga)
        for i, (x, y) in enumerate(zip(a, b)):
            assert np.array_equal(x, y), f"replay {k}: tensor {i} differs from the eager step"


def test_overlapped_step_matches_sequential_step():
    """Eager: AdamW on a second stream beside the Muon step (ma_muon_adamw_step)
    gives the bits of the Muon step followed by the AdamW step, over 3 steps."""
    need_gpu()
    import adamw_optimizer_step_amd as M
    init_m, init_a = _state(5)
    outs = []
    for overlap in (False, True):
        dm, da = _to_dev(init_m, init_a)
        groups, hp, _ = _stepper(M, dm, da, None)
        ws = torch.empty(max(1, M.muon_workspace_size(groups, hp)), dtype=torch.uint8, device=DEV)
        _, _, step = _stepper(M, dm, da, ws, overlap=overlap)
        for _k in range(3):
            step()
        torch.cuda.synchronize()
        outs.append(_snapshot(dm, da))
    say("overlapped vs sequential eager steps")
    for a, b in zip(*outs):
        assert np.array_equal(a, b)



@pytest.mark.parametrize("captured", [False, True])
def test_failure_after_fork_still_joins(captured):
    """A launch failing after the fork (forced by the library's test hook)
    returns the error, but the caller's stream still waits for the AdamW work
    already queued on the side stream: eagerly, AdamW is complete once the
    caller's stream is synchronised; in a graph capture, the capture ends
    normally (a side stream left unjoined would make it fail)."""
    need_gpu()
    import adamw_optimizer_step_amd as M
    import oracle as O
    from adamw_optimizer_step_amd import _lib as L
    init_m, init_a = _state(9)
    dm, da = _to_dev(init_m, init_a)
    groups, hp, _ = _stepper(M, dm, da, None)
    ws = torch.empty(max(1, M.muon_workspace_size(groups, hp)), dtype=torch.uint8, device=DEV)
    _, _, step = _stepper(M, dm, da, ws, overlap=True)
    say("failure after the fork", "captured" if captured else "eager")
    if captured:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            L.check(L.lib().ma_test_fail_after_fork())
            with pytest.raises(M.MuonAdamWError) as err:
                step()
        assert err.value.status == L.MA_ERR_HIP
        torch.cuda.synchronize()
        return
    L.check(L.lib().ma_test_fail_after_fork())
    with pytest.raises(M.MuonAdamWError) as err:
        step()
    assert err.value.status == L.MA_ERR_HIP and "injected" in str(err.value)
    torch.cuda.current_stream(DEV).synchronize()
    p, g, m, v = (t.numpy() for t in init_a)
    ep, em, ev = O.adamw_step(p, g, m, v, 7, lr=float(np.float32(3e-4)), beta1=float(np.float32(0.9)),
                              beta2=float(np.float32(0.95)), eps=float(np.float32(1e-8)),
                              weight_decay=float(np.float32(0.1)))
    for got, exp in ((da[0], ep), (da[2], em), (da[3], ev)):
        assert np.array_equal(got.cpu().numpy().view(np.uint32), exp.view(np.uint32))
    torch.cuda.synchronize()
