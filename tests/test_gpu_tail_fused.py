"""latent_moe_tail_fused: the latent-MoE tail with the up-projection's K-split
sum inside its launch.

Where latent_moe_tail splits the GEMM's K in two on the 4-wave MFMA tile and
then sums the splits in a second launch (17 <= M <= 64 at the Kimi-K3 shapes),
the second split's workgroups read the first split's fp32 sums, each stored
with the call's generation, add them first and store bf16(sum + shared): the
reduction launch's order, so the outputs equal latent_moe_tail's bit for bit.
Elsewhere the call is latent_moe_tail.  Both are checked against the oracle.
One workspace, zero-filled once, serves calls of changing shapes, graph
replays, in-place calls and guard margins.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bf16_skinny_gemm_02_amd as sg
import oracle
import synth
from tests.gpu_util import assert_close, dev, host, nan_like

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _eq(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _ws(M, device, D=synth.D_HIDDEN, d=synth.D_LATENT):
    return torch.zeros(sg.sg_workspace_bytes(sg.SG_OP_LATENT_TAIL_FUSED, M, D, d), dtype=torch.uint8,
                       device=device)


@pytest.mark.parametrize("M", [1, 8, 16, 17, 24, 32, 33, 48, 63, 64, 65, 130])
def test_tail_fused_equals_tail_and_oracle(device, M):
    cfg = sg.sg_select(M, synth.D_HIDDEN, synth.D_LATENT)
    _say(f"latent_moe_tail_fused M={M} cfg={cfg}")
    L, gamma, w_up, S = synth.tail_inputs(M, seed=5000 + M)
    args = [dev(a, device) for a in (L, gamma, w_up, S)]
    f = sg.latent_moe_tail_fused(*args, out=nan_like((M, synth.D_HIDDEN), device),
                                 workspace=_ws(M, device))
    t = sg.latent_moe_tail(*args)
    torch.cuda.synchronize()
    assert _eq(f, t)
    ex, _ = oracle.latent_tail(L, gamma, 1e-6, w_up, S)
    assert_close(host(f), ex, f"fused tail M={M}")


@pytest.mark.parametrize("M", [20, 64])
def test_tail_fused_no_shared_and_inplace(device, M):
    L, gamma, w_up, S = synth.tail_inputs(M, seed=5100 + M)
    Ld, gd, wd = dev(L, device), dev(gamma, device), dev(w_up, device)
    ws = _ws(M, device)
    out = sg.latent_moe_tail_fused(Ld, gd, wd, None, eps=1e-5, workspace=ws)
    inplace = dev(S, device).clone()
    sg.latent_moe_tail_fused(Ld, gd, wd, inplace, eps=1e-5, out=inplace, workspace=ws)
    torch.cuda.synchronize()
    assert _eq(out, sg.latent_moe_tail(Ld, gd, wd, None, eps=1e-5))
    ex, _ = oracle.latent_tail(L, gamma, 1e-5, w_up, None)
    assert_close(host(out), ex, "fused tail without shared")
    ex_s, _ = oracle.latent_tail(L, gamma, 1e-5, w_up, S)
    assert_close(host(inplace), ex_s, "fused tail in place")


def test_tail_fused_one_workspace_across_shapes(device):
    """One workspace, zero-filled once, for a sequence of calls whose tile
    counts and paths change (the in-launch sum at 17..64, the wave-split fold
    at 8, the block tile and its reduction launch at 130, the GEMV at 1):
    every call must equal latent_moe_tail, so the generations never fall out
    of step."""
    seq = [17, 64, 8, 32, 17, 130, 48, 1, 64, 33]
    ws = torch.zeros(max(_ws(M, device).numel() for M in seq), dtype=torch.uint8, device=device)
    for i, M in enumerate(seq):
        _say(f"shared workspace call {i}: M={M}")
        L, gamma, w_up, S = synth.tail_inputs(M, seed=5200 + i)
        args = [dev(a, device) for a in (L, gamma, w_up, S)]
        a = sg.latent_moe_tail_fused(*args, workspace=ws)
        b = sg.latent_moe_tail(*args)
        torch.cuda.synchronize()
        assert _eq(a, b), M


@pytest.mark.parametrize("M", [17, 64])
def test_tail_fused_graph_replay(device, M):
    """Capture the fused tail in a graph, replay it several times with eager
    work in between (the output reset to NaN before each replay), and compare
    every replay bit for bit with the eager result."""
    L, gamma, w_up, S = synth.tail_inputs(M, seed=5300 + M)
    args = [dev(a, device) for a in (L, gamma, w_up, S)]
    eager = sg.latent_moe_tail(*args)
    out = torch.empty_like(eager)
    ws = _ws(M, device)
    side = torch.cuda.Stream(device)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            sg.latent_moe_tail_fused(*args, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.ones(4096, device=device).sum()
        torch.cuda.synchronize()
        assert _eq(out, eager), f"replay {rep}"
        del junk


@pytest.mark.parametrize("M", [17, 50])
def test_tail_fused_writes_only_its_output(device, M):
    from tests.test_gpu_guards import Guarded, GuardedWs
    L, gamma, w_up, S = synth.tail_inputs(M, seed=5400 + M)
    out = Guarded(M, synth.D_HIDDEN, device)
    ws = GuardedWs(_ws(M, device).numel(), device)
    sg.latent_moe_tail_fused(dev(L, device), dev(gamma, device), dev(w_up, device), dev(S, device),
                             out=out.view, workspace=ws.view)
    torch.cuda.synchronize()
    out.check("fused tail out")
    ws.check("fused tail workspace")
    ex, _ = oracle.latent_tail(L, gamma, 1e-6, w_up, S)
    assert_close(out.bits(), ex, "guarded fused tail")


def test_tail_fused_zero_weights_is_shared(device):
    """Zero up-projection weights: every sum is exactly zero, so the fused
    tail must return the shared-expert partial bit for bit (the in-launch
    sum adds the first split's zeros to the second's)."""
    M = 40
    L, gamma, w_up, S = synth.tail_inputs(M, seed=5500)
    zero_w = np.zeros_like(w_up)
    out = sg.latent_moe_tail_fused(dev(L, device), dev(gamma, device), dev(zero_w, device), dev(S, device),
                                   workspace=_ws(M, device))
    torch.cuda.synchronize()
    assert np.array_equal(host(out), S)


def test_tail_fused_timeout_gives_nan_and_recovers(device):
    """The second split's wait is bounded: with a header whose generations
    never match, the call still returns with NaN outputs; zero-filling the
    header again restores latent_moe_tail's results."""
    M = 24
    L, gamma, w_up, S = synth.tail_inputs(M, seed=5600)
    args = [dev(a, device) for a in (L, gamma, w_up, S)]
    ws = _ws(M, device)
    hdr = ws[:sg._lib.SG_FAB_HEADER_BYTES].view(torch.int32)
    hdr[4096:].fill_(1000)  # consumers wait for 1001; producers tag 1
    out = sg.latent_moe_tail_fused(*args, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    ws.zero_()
    out2 = sg.latent_moe_tail_fused(*args, workspace=ws)
    torch.cuda.synchronize()
    assert _eq(out2, sg.latent_moe_tail(*args))
