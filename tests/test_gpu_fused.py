"""kda_fab_fb_proj_fused: the F_A/beta -> F_B branch as one launch.

The F_A/beta workgroups hand their split-K partials to F_B workgroups of the
same grid through flags in the workspace header (the role of the
programmatic dependent launch that chains the two GEMMs of run_fab_fb in
"Overlap low-M TP8 KDA projections").  It runs the same F_A/beta kernel code
over the same K-ranges and sums the partials in the same order as
kda_fab_fb_proj, so the two must agree bit for bit; both are checked against
the oracle.  One workspace, zero-filled once, serves calls of changing shapes
(the header keeps itself consistent), graph replays, and guard margins.
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


def _ws(M, n_ab, K=synth.HIDDEN, device=None, extra=0):
    return torch.zeros(sg.sg_workspace_bytes(sg.SG_OP_FAB_FB, M, n_ab, K) + extra, dtype=torch.uint8,
                       device=device)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 13, 16, 17, 64])
@pytest.mark.parametrize("n_ab", [136, 144])
def test_fused_equals_two_launches_and_oracle(device, M, n_ab):
    cfg = sg.sg_kda_select(sg.SG_KDA_FAB_ALONE, M, synth.HIDDEN, 0, n_ab)
    _say(f"kda_fab_fb_proj_fused M={M} n_ab={n_ab} cfg={cfg}")
    x, w_ab, w_b = synth.fab_fb_inputs(M, seed=900 + M, n_ab=n_ab)
    xd, ad, bd = dev(x, device), dev(w_ab, device), dev(w_b, device)
    g1_f, beta_f, fa_f = sg.kda_fab_fb_proj_fused(xd, ad, bd, want_f_a=True,
                                                  beta=nan_like((M, n_ab - 128), device),
                                                  g1=nan_like((M, synth.N_B), device),
                                                  workspace=_ws(M, n_ab, device=device))
    g1_t, beta_t, fa_t = sg.kda_fab_fb_proj(xd, ad, bd, want_f_a=True)
    torch.cuda.synchronize()
    for a, b, n in ((g1_f, g1_t, "g1"), (beta_f, beta_t, "beta"), (fa_f, fa_t, "f_a")):
        assert _eq(a, b), n
    o = oracle.fab_fb(x, w_ab, w_b)
    assert_close(host(g1_f), o["g1_exact"], "fused g1")
    assert_close(host(beta_f), o["beta_exact"], "fused beta")
    assert_close(host(fa_f), o["p_exact"][:, :128], "fused f_a")


@pytest.mark.parametrize("M", [1, 8])
def test_fused_lattice_bitwise(device, M):
    K, n_ab = synth.HIDDEN, 136
    x = synth.lattice_activation((M, K), seed=1500 + M)
    w_ab = synth.lattice_weight((n_ab, K), seed=1600 + M)
    w_b = synth.lattice_weight((1024, 128), seed=1700 + M)
    g1, beta, f_a = sg.kda_fab_fb_proj_fused(dev(x, device), dev(w_ab, device), dev(w_b, device),
                                             want_f_a=True)
    torch.cuda.synchronize()
    o = oracle.fab_fb(x, w_ab, w_b)
    assert np.array_equal(host(f_a), o["f_a"])
    assert np.array_equal(host(beta), o["beta"])
    assert np.array_equal(host(g1), o["g1_bits"])


def test_fused_one_workspace_across_shapes(device):
    """One workspace, zero-filled once, for a sequence of calls whose producer
    and consumer counts change (GEMV at M = 1, wave-split at 2..16 with
    different splits, the two-launch fallback at 40): every call must equal
    the two-launch result, so the flags never fall out of step."""
    seq = [(1, 136), (8, 136), (2, 144), (16, 136), (40, 136), (1, 144), (4, 136), (13, 144), (1, 136)]
    ws = torch.zeros(max(sg.sg_workspace_bytes(sg.SG_OP_FAB_FB, M, n, synth.HIDDEN) for M, n in seq),
                     dtype=torch.uint8, device=device)
    for i, (M, n_ab) in enumerate(seq):
        _say(f"shared workspace call {i}: M={M} n_ab={n_ab}")
        x, w_ab, w_b = synth.fab_fb_inputs(M, seed=2000 + i, n_ab=n_ab)
        xd, ad, bd = dev(x, device), dev(w_ab, device), dev(w_b, device)
        g1_f, beta_f = sg.kda_fab_fb_proj_fused(xd, ad, bd, workspace=ws)
        g1_t, beta_t = sg.kda_fab_fb_proj(xd, ad, bd)
        torch.cuda.synchronize()
        assert _eq(g1_f, g1_t) and _eq(beta_f, beta_t), (M, n_ab)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_fused_graph_replay(device, M):
    x, w_ab, w_b = synth.fab_fb_inputs(M, seed=2100 + M)
    xd, ad, bd = dev(x, device), dev(w_ab, device), dev(w_b, device)
    g1_e, beta_e = sg.kda_fab_fb_proj(xd, ad, bd)
    g1 = torch.empty_like(g1_e)
    beta = torch.empty_like(beta_e)
    ws = _ws(M, 136, device=device)
    side = torch.cuda.Stream(device)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            sg.kda_fab_fb_proj_fused(xd, ad, bd, g1=g1, beta=beta, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        g1.fill_(float("nan"))
        beta.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.ones(4096, device=device).sum()
        torch.cuda.synchronize()
        assert _eq(g1, g1_e) and _eq(beta, beta_e), f"replay {rep}"
        del junk


@pytest.mark.parametrize("M", [1, 3, 16])
def test_fused_writes_only_its_outputs(device, M):
    from tests.test_gpu_guards import Guarded, GuardedWs
    x, w_ab, w_b = synth.fab_fb_inputs(M, seed=2200 + M, n_ab=141)
    beta = Guarded(M, 13, device)
    g1 = Guarded(M, synth.N_B, device)
    f_a = Guarded(M, 128, device)
    ws = GuardedWs(sg.sg_workspace_bytes(sg.SG_OP_FAB_FB, M, 141, synth.HIDDEN), device)
    sg.kda_fab_fb_proj_fused(dev(x, device), dev(w_ab, device), dev(w_b, device), f_a=f_a.view,
                             beta=beta.view, g1=g1.view, workspace=ws.view)
    torch.cuda.synchronize()
    for t, n in ((beta, "beta"), (g1, "g1"), (f_a, "f_a"), (ws, "workspace")):
        t.check(f"fused {n}")
    o = oracle.fab_fb(x, w_ab, w_b)
    assert_close(g1.bits(), o["g1_exact"], "guarded fused g1")


@pytest.mark.parametrize("M", [1, 4])
def test_fused_timeout_gives_nan_and_recovers(device, M):
    """The F_B workgroups' wait is bounded: with a header whose generations
    never match, the call still returns with NaN g1 and beta; zero-filling
    the header again restores the two-launch results."""
    x, w_ab, w_b = synth.fab_fb_inputs(M, seed=2300 + M)
    xd, ad, bd = dev(x, device), dev(w_ab, device), dev(w_b, device)
    ws = _ws(M, 136, device=device)
    ws[:sg._lib.SG_FAB_HEADER_BYTES].view(torch.int32)[4096:].fill_(1000)
    g1, beta = sg.kda_fab_fb_proj_fused(xd, ad, bd, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(g1.float()).all() and torch.isnan(beta.float()).all()
    ws.zero_()
    g1b, betab = sg.kda_fab_fb_proj_fused(xd, ad, bd, workspace=ws)
    g1_t, beta_t = sg.kda_fab_fb_proj(xd, ad, bd)
    torch.cuda.synchronize()
    assert _eq(g1b, g1_t) and _eq(betab, beta_t)
