"""kda_projection_fused: the KDA projection as one launch.

The F_A/beta -> F_B chain that "Overlap low-M TP8 KDA projections" runs on an
auxiliary stream beside the Q/K/V/G GEMM rides inside the Q/K/V/G launch: a
fifth wave of every wave-split workgroup computes a slice of P = x W_ab^T
(fp32 partials, each stored with the call's generation) and the fifth waves of
the next workgroups read them until all carry it, sum them in fixed order and
compute g1.  qkvg,
beta and g1 are checked against the oracle; on integer-lattice inputs every
partial sum is exact, so all three must equal the oracle bit for bit.  One
workspace, zero-filled once, serves calls of changing shapes (the header keeps
itself consistent), graph replays, and guard margins; shapes the helper
geometry does not fit take the one-stream schedule.
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


def _ws(M, K=synth.HIDDEN, n_qkvg=4096, n_ab=136, device=None):
    return torch.zeros(sg.sg_kda_workspace_bytes(sg.SG_KDA_ONE_LAUNCH, M, K, n_qkvg, n_ab),
                       dtype=torch.uint8, device=device)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 9, 12, 15, 16, 17, 24])
def test_one_launch_matches_oracle(device, M):
    _say(f"kda_projection_fused M={M}")
    x, packed, w_b = synth.overlap_inputs(M, seed=3000 + M)
    xd, pd, wbd = dev(x, device), dev(packed, device), dev(w_b, device)
    q, g1, beta = sg.kda_projection_fused(xd, pd, wbd, qkvg=nan_like((M, 4096), device),
                                          beta=nan_like((M, 8), device),
                                          g1=nan_like((M, synth.N_B), device), workspace=_ws(M, device=device))
    torch.cuda.synchronize()
    o = oracle.projection_overlap(x, packed, w_b)
    assert_close(host(q), o["qkvg_exact"], "qkvg")
    assert_close(host(g1), o["g1_exact"], "g1")
    assert_close(host(beta), o["beta_exact"], "beta")
    if not sg.sg_kda_one_launch_fits(M, synth.HIDDEN, 4096, 136, 128, synth.N_B):  # one-stream schedule
        q_s, g1_s, b_s = sg.kda_projection_overlap(xd, pd, wbd)
        torch.cuda.synchronize()
        assert _eq(q, q_s) and _eq(g1, g1_s) and _eq(beta, b_s)


@pytest.mark.parametrize("M,K", [(2, 7168), (8, 7168), (5, 7168), (12, 7168), (16, 7168), (3, 4096),
                                 (7, 1032), (13, 1032)])
def test_one_launch_lattice_bitwise(device, M, K):
    """Integer-lattice inputs: every partial sum is exact in fp32, so qkvg,
    beta and g1 must equal the oracle bit for bit whatever the K-ranges,
    the order of the sums or the host that formed f_a.  K = 4096 and 1032
    give other producer counts (fewer K-ranges; one K-range that ends
    inside a 512-k step); M = 12, 13 and 16 have two groups of activation
    rows."""
    _say(f"kda_projection_fused lattice M={M} K={K}")
    x = synth.lattice_activation((M, K), seed=3100 + M)
    packed = synth.lattice_weight((4096 + 136, K), seed=3200 + M)
    w_b = synth.lattice_weight((1024, 128), seed=3300 + M)
    q, g1, beta = sg.kda_projection_fused(dev(x, device), dev(packed, device), dev(w_b, device),
                                          workspace=_ws(M, K, device=device))
    torch.cuda.synchronize()
    o = oracle.projection_overlap(x, packed, w_b)
    assert np.array_equal(host(q), o["qkvg_bits"])
    assert np.array_equal(host(beta), o["beta"])
    assert np.array_equal(host(g1), o["g1_bits"])


def test_one_launch_one_workspace_across_shapes(device):
    """One workspace, zero-filled once, for a sequence of calls of changing M
    (one launch at 1..16, the one-stream schedule at 17 and 40): every call
    must equal a call on a fresh workspace, so the flags never fall out of
    step."""
    seq = [2, 8, 16, 1, 4, 40, 3, 9, 17, 2, 13]
    ws = torch.zeros(max(_ws(M).numel() for M in seq), dtype=torch.uint8, device=device)
    for i, M in enumerate(seq):
        _say(f"shared workspace call {i}: M={M}")
        x, packed, w_b = synth.overlap_inputs(M, seed=3400 + i)
        xd, pd, wbd = dev(x, device), dev(packed, device), dev(w_b, device)
        a = sg.kda_projection_fused(xd, pd, wbd, workspace=ws)
        b = sg.kda_projection_fused(xd, pd, wbd, workspace=_ws(M, device=device))
        torch.cuda.synchronize()
        for u, v, n in zip(a, b, ("qkvg", "g1", "beta")):
            assert _eq(u, v), (M, n)


@pytest.mark.parametrize("M", [2, 8, 12, 16])
def test_one_launch_graph_replay(device, M):
    """Capture the one-launch projection in a graph, replay it several times
    with eager work in between (outputs reset to NaN before each replay), and
    compare every replay bit for bit with the eager result."""
    _say(f"kda_projection_fused graph M={M}")
    x, packed, w_b = synth.overlap_inputs(M, seed=3500 + M)
    xd, pd, wbd = dev(x, device), dev(packed, device), dev(w_b, device)
    q_e, g1_e, b_e = sg.kda_projection_fused(xd, pd, wbd)
    q = torch.empty_like(q_e)
    g1 = torch.empty_like(g1_e)
    beta = torch.empty_like(b_e)
    ws = _ws(M, device=device)
    side = torch.cuda.Stream(device)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            sg.kda_projection_fused(xd, pd, wbd, qkvg=q, g1=g1, beta=beta, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        for t in (q, g1, beta):
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.ones(4096, device=device).sum()
        torch.cuda.synchronize()
        assert _eq(q, q_e) and _eq(g1, g1_e) and _eq(beta, b_e), f"replay {rep}"
        del junk


@pytest.mark.parametrize("M", [2, 7, 10, 13])
def test_one_launch_writes_only_its_outputs(device, M):
    from tests.test_gpu_guards import Guarded, GuardedWs
    x, packed, w_b = synth.overlap_inputs(M, seed=3600 + M)
    q = Guarded(M, 4096, device)
    beta = Guarded(M, 8, device)
    g1 = Guarded(M, synth.N_B, device)
    ws = GuardedWs(_ws(M).numel(), device)
    sg.kda_projection_fused(dev(x, device), dev(packed, device), dev(w_b, device), qkvg=q.view,
                            beta=beta.view, g1=g1.view, workspace=ws.view)
    torch.cuda.synchronize()
    for t, n in ((q, "qkvg"), (beta, "beta"), (g1, "g1"), (ws, "workspace")):
        t.check(f"one-launch {n}")
    o = oracle.projection_overlap(x, packed, w_b)
    assert_close(q.bits(), o["qkvg_exact"], "guarded qkvg")
    assert_close(g1.bits(), o["g1_exact"], "guarded g1")
    assert_close(beta.bits(), o["beta_exact"], "guarded beta")


def _desync(ws):
    """A header whose cursors are far ahead of its flags: every waiter's
    generation (its cursor + 1) is one no producer of the next call stores
    (its flag + 1), so each bounded wait runs to its limit."""
    hdr = ws[:sg._lib.SG_FAB_HEADER_BYTES].view(torch.int32)
    hdr[:4096].zero_()
    hdr[4096:].fill_(1000)


def test_one_launch_timeout_gives_nan_and_recovers(device):
    """The hosts' wait is bounded: with a header whose generations never
    match, the call still returns, qkvg (which does not wait) is right, and
    g1 and beta are NaN; zero-filling the header again restores the results."""
    M = 4
    x, packed, w_b = synth.overlap_inputs(M, seed=3700)
    xd, pd, wbd = dev(x, device), dev(packed, device), dev(w_b, device)
    ws = _ws(M, device=device)
    _desync(ws)
    q, g1, beta = sg.kda_projection_fused(xd, pd, wbd, workspace=ws)
    torch.cuda.synchronize()
    o = oracle.projection_overlap(x, packed, w_b)
    assert_close(host(q), o["qkvg_exact"], "qkvg after a time-out")
    assert torch.isnan(g1.float()).all() and torch.isnan(beta.float()).all()
    ws.zero_()
    q2, g2, b2 = sg.kda_projection_fused(xd, pd, wbd, workspace=ws)
    torch.cuda.synchronize()
    assert_close(host(g2), o["g1_exact"], "g1 after re-zeroing")
    assert_close(host(b2), o["beta_exact"], "beta after re-zeroing")
