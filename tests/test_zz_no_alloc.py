"""kda_projection_noalloc: the KDA projection with its workspaces in the
library's own per-GPU device array, for callers that cannot allocate.

Called through the C ABI (the binding only marshals), compared bit for bit
with kda_projection_overlap on the same inputs (same kernels, same
configurations, so the same bits), on two calls in a row whose second input
is smaller, so the second call runs on an array that still holds the first
call's contents; once more inside a captured graph.
"""
from __future__ import annotations

import pytest
import torch

import bf16_skinny_gemm_02_amd as sg
import oracle
import synth
from tests.gpu_util import assert_close, dev, host

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _outputs(M, device):
    return (torch.full((M, synth.N_QKVG), float("nan"), dtype=torch.bfloat16, device=device),
            torch.full((M, synth.N_B), float("nan"), dtype=torch.bfloat16, device=device),
            torch.full((M, synth.N_AB - synth.RANK), float("nan"), dtype=torch.bfloat16,
                       device=device))


def _equal(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("ms", [(64, 4), (16, 1), (100, 17)])
def test_noalloc_matches_overlap_on_two_calls(device, ms):
    for M in ms:  # the second call is smaller than the first
        _say(f"kda_projection_noalloc M={M} (sequence {ms})")
        x, packed, w_b = synth.overlap_inputs(M, seed=700 + M)
        xd, pd, wbd = dev(x, device), dev(packed, device), dev(w_b, device)
        q, g1, beta = _outputs(M, device)
        sg.kda_projection_noalloc(xd, pd, wbd, qkvg=q, g1=g1, beta=beta)
        q_r, g1_r, beta_r = sg.kda_projection_overlap(xd, pd, wbd)
        torch.cuda.synchronize()
        for a, b, n in ((q, q_r, "qkvg"), (g1, g1_r, "g1"), (beta, beta_r, "beta")):
            assert _equal(a, b), f"{n} M={M}"
        o = oracle.projection_overlap(x, packed, w_b)
        assert_close(host(g1), o["g1_exact"], f"noalloc g1 M={M}")
        assert_close(host(beta), o["beta_exact"], f"noalloc beta M={M}")


def test_noalloc_two_streams_and_graph(device):
    """The fork/join schedule on the library's array, and the single-stream
    call captured in a graph and replayed: both equal the eager result."""
    M = 8
    x, packed, w_b = synth.overlap_inputs(M, seed=808)
    xd, pd, wbd = dev(x, device), dev(packed, device), dev(w_b, device)
    q_r, g1_r, beta_r = sg.kda_projection_overlap(xd, pd, wbd)
    q, g1, beta = _outputs(M, device)
    aux = torch.cuda.Stream(device)
    sg.kda_projection_noalloc(xd, pd, wbd, qkvg=q, g1=g1, beta=beta, aux_stream=aux,
                              fork=sg.HipEvent(), join=sg.HipEvent())
    torch.cuda.synchronize()
    for a, b in ((q, q_r), (g1, g1_r), (beta, beta_r)):
        assert _equal(a, b)
    q, g1, beta = _outputs(M, device)
    side = torch.cuda.Stream(device)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            sg.kda_projection_noalloc(xd, pd, wbd, qkvg=q, g1=g1, beta=beta)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        for t in (q, g1, beta):
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for a, b in ((q, q_r), (g1, g1_r), (beta, beta_r)):
            assert _equal(a, b), f"replay {rep}"


def test_noalloc_rejects_shapes_beyond_its_array(device):
    # a wide F_A/beta block at M = 256: 4 x 256 x 2304 fp32 partials beside the
    # Q/K/V/G ones, 17 MiB in all
    M, K, nq, nab = 256, 7168, 4096, 2304
    need = (sg.sg_kda_workspace_bytes(0, M, K, nq, nab) +
            sg.sg_kda_workspace_bytes(1, M, K, nq, nab))
    assert need > sg._lib.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=device)
    pw = torch.zeros((nq + nab, K), dtype=torch.bfloat16, device=device)
    wb = torch.zeros((1024, 128), dtype=torch.bfloat16, device=device)
    q = torch.zeros((M, nq), dtype=torch.bfloat16, device=device)
    g1 = torch.zeros((M, 1024), dtype=torch.bfloat16, device=device)
    beta = torch.zeros((M, nab - 128), dtype=torch.bfloat16, device=device)
    with pytest.raises(ValueError, match="workspace"):
        sg.kda_projection_noalloc(x, pw, wb, n_qkvg=nq, n_ab=nab, qkvg=q, g1=g1, beta=beta)
