"""Write safety of every entry point, and shapes that alternate inside one graph.

Guard canaries: each output and workspace is a window of a larger buffer whose
margins (and, for a strided output, the gaps between its rows) hold a fixed
sentinel.  After the call every sentinel must be unchanged bit for bit, so a
store past an output or a workspace fails even when every output element is
right.  Outputs start as NaN, so an element left unwritten fails too.  The
packed 8- and 16-byte stores of the kernels are exercised with N % 4 != 0,
odd row strides and an in-place residual.

Alternating shapes: one captured graph holds calls at M = 1, 64, 4, 17 and 256
(the GEMV, wave-split, split-K tile and block paths) on shared activation
buffers and one shared workspace per entry point, replayed several times and
compared with the same sequence run eagerly.  This is where per-device
launch state, segment selection or a workspace reused across shapes could go
wrong.  (The pages' own tests for the fused GEMM + reduce-scatter kernel use
non-aligned M, alternating shapes and graph capture; an uninitialised output
once went unnoticed there, which is why outputs start as NaN.)
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bf16_skinny_gemm_02_amd as sg
import oracle
import synth
from tests.gpu_util import assert_close, dev, host

pytestmark = pytest.mark.gpu

MARGIN = 4096            # elements of sentinel before and after each window
SENT16 = 0x7FA5          # a NaN payload no kernel produces (bf16 outputs)
SENT8 = 0xA5             # workspace margins


def _say(*a):
    print(*a, flush=True)


class Guarded:
    """A bf16 [rows, cols] window (row stride ld >= cols) inside a sentinel
    buffer; the window starts as NaN, everything else as SENT16."""

    def __init__(self, rows, cols, device, ld=None, init=None):
        self.rows, self.cols = rows, cols
        self.ld = cols if ld is None else ld
        span = (rows - 1) * self.ld + cols if rows > 0 else 0
        n = MARGIN + span + MARGIN
        self.buf = torch.full((n,), SENT16, dtype=torch.int16, device=device)
        self.view = self.buf.as_strided((rows, cols), (self.ld, 1), MARGIN).view(torch.bfloat16)
        if init is None:
            self.view.fill_(float("nan"))
        else:
            self.view.copy_(init)
        mask = np.ones(n, dtype=bool)
        for r in range(rows):
            mask[MARGIN + r * self.ld: MARGIN + r * self.ld + cols] = False
        self.mask = mask

    def check(self, what):
        b = self.buf.cpu().numpy().view(np.uint16)
        bad = np.flatnonzero(self.mask & (b != SENT16))
        assert bad.size == 0, (f"{what}: {bad.size} sentinel elements overwritten, first at "
                               f"offset {bad[:4] - MARGIN} relative to the window")

    def bits(self):
        return host(self.view)


class GuardedWs:
    """A zero-filled workspace of `nbytes` inside 0xA5 margins."""

    def __init__(self, nbytes, device):
        self.n = nbytes
        self.buf = torch.full((MARGIN + nbytes + MARGIN,), SENT8, dtype=torch.uint8, device=device)
        self.buf[MARGIN:MARGIN + nbytes].zero_()
        # 256-byte aligned window start (MARGIN is a multiple of 256)
        self.view = self.buf[MARGIN:MARGIN + nbytes] if nbytes else None

    def check(self, what):
        b = self.buf.cpu().numpy()
        bad = np.concatenate([np.flatnonzero(b[:MARGIN] != SENT8),
                              MARGIN + self.n + np.flatnonzero(b[MARGIN + self.n:] != SENT8)])
        assert bad.size == 0, f"{what}: workspace margin overwritten at byte {bad[:4] - MARGIN}"


GEMM_GUARD_CASES = [
    # (M, N, K, residual, ldc): GEMV row / split-K, small-K, wave-split, tile, block; N % 4 != 0
    # and odd row strides make the packed stores fall back to element stores at the edges
    (1, 1029, 2048, True, 1029), (1, 77, 7168, False, 79), (5, 61, 128, True, 67),
    (3, 1030, 1000, True, 1031), (8, 4099, 7168, False, 4101), (16, 515, 2056, True, 515),
    (17, 301, 1000, True, 305), (33, 1027, 4104, False, 1027), (64, 129, 2048, True, 131),
    (100, 77, 4104, False, 81), (256, 203, 520, True, 203), (24, 7171, 2048, True, 7173),
]


@pytest.mark.parametrize("M,N,K,res,ldc", GEMM_GUARD_CASES)
def test_skinny_gemm_writes_only_its_output(device, M, N, K, res, ldc):
    _say(f"guard skinny_gemm M={M} N={N} K={K} res={res} ldc={ldc} cfg={sg.sg_select(M, N, K, res)}")
    A, W, R = synth.gemm_inputs(M, N, K, seed=31 * M + N + K, residual=res)
    out = Guarded(M, N, device, ld=ldc)
    ws = GuardedWs(sg.sg_workspace_bytes(sg.SG_OP_GEMM, M, N, K), device)
    sg.skinny_gemm(dev(A, device), dev(W, device), dev(R, device) if res else None, out=out.view,
                   workspace=ws.view)
    torch.cuda.synchronize()
    out.check("skinny_gemm output")
    ws.check("skinny_gemm workspace")
    assert_close(out.bits(), oracle.gemm(A, W, R)[0], "guarded skinny_gemm")


@pytest.mark.parametrize("M,N,K", [(4, 1027, 1000), (17, 301, 2056), (100, 515, 1032),
                                   (1, 1029, 2048)])
def test_skinny_gemm_inplace_residual_writes_only_its_output(device, M, N, K):
    _say(f"guard in-place skinny_gemm M={M} N={N} K={K}")
    A, W, R = synth.gemm_inputs(M, N, K, seed=7 * M + N, residual=True)
    c = Guarded(M, N, device, init=dev(R, device))
    ws = GuardedWs(sg.sg_workspace_bytes(sg.SG_OP_GEMM, M, N, K), device)
    sg.skinny_gemm(dev(A, device), dev(W, device), c.view, out=c.view, workspace=ws.view)
    torch.cuda.synchronize()
    c.check("in-place output")
    ws.check("in-place workspace")
    assert_close(c.bits(), oracle.gemm(A, W, R)[0], "guarded in-place")


@pytest.mark.parametrize("M", [1, 3, 8, 16, 17, 64, 100])
@pytest.mark.parametrize("n_ab", [136, 141])
def test_fab_fb_writes_only_its_outputs(device, M, n_ab):
    _say(f"guard kda_fab_fb_proj M={M} n_ab={n_ab}")
    x, w_ab, w_b = synth.fab_fb_inputs(M, seed=50 + M, n_ab=n_ab)
    beta = Guarded(M, n_ab - 128, device)
    g1 = Guarded(M, synth.N_B, device)
    f_a = Guarded(M, 128, device)
    ws = GuardedWs(sg.sg_workspace_bytes(sg.SG_OP_FAB_FB, M, n_ab, synth.HIDDEN), device)
    sg.kda_fab_fb_proj(dev(x, device), dev(w_ab, device), dev(w_b, device), f_a=f_a.view,
                       beta=beta.view, g1=g1.view, workspace=ws.view)
    torch.cuda.synchronize()
    for t, n in ((beta, "beta"), (g1, "g1"), (f_a, "f_a"), (ws, "workspace")):
        t.check(f"kda_fab_fb_proj {n}")
    o = oracle.fab_fb(x, w_ab, w_b)
    assert_close(g1.bits(), o["g1_exact"], "guarded g1")
    assert_close(beta.bits(), o["beta_exact"], "guarded beta")
    assert_close(f_a.bits(), o["p_exact"][:, :128], "guarded f_a")


@pytest.mark.parametrize("concurrent", [False, True])
@pytest.mark.parametrize("M", [1, 4, 13, 17, 64, 100])
def test_projection_writes_only_its_outputs(device, M, concurrent):
    _say(f"guard kda_projection_overlap M={M} concurrent={concurrent}")
    K = synth.HIDDEN
    x, packed, w_b = synth.overlap_inputs(M, seed=60 + M)
    q = Guarded(M, synth.N_QKVG, device)
    beta = Guarded(M, 8, device)
    g1 = Guarded(M, synth.N_B, device)
    wsm = GuardedWs(sg.sg_kda_workspace_bytes(0, M, K, 4096, 136), device)
    wsa = GuardedWs(sg.sg_kda_workspace_bytes(1, M, K, 4096, 136), device)
    kw = {}
    if concurrent:
        kw = dict(aux_stream=torch.cuda.Stream(device), fork=sg.HipEvent(), join=sg.HipEvent())
    sg.kda_projection_overlap(dev(x, device), dev(packed, device), dev(w_b, device), qkvg=q.view,
                              beta=beta.view, g1=g1.view, ws_main=wsm.view, ws_aux=wsa.view, **kw)
    torch.cuda.synchronize()
    for t, n in ((q, "qkvg"), (beta, "beta"), (g1, "g1"), (wsm, "ws_main"), (wsa, "ws_aux")):
        t.check(f"projection {n}")
    o = oracle.projection_overlap(x, packed, w_b)
    assert_close(q.bits(), o["qkvg_exact"], "guarded qkvg")
    assert_close(g1.bits(), o["g1_exact"], "guarded g1")
    assert_close(beta.bits(), o["beta_exact"], "guarded beta")


@pytest.mark.parametrize("M,d,D,inplace", [(1, 2048, 7168, False), (4, 2048, 7171, True),
                                           (16, 2048, 7168, False), (17, 2048, 7168, True),
                                           (64, 1032, 3001, False), (256, 2048, 7168, True),
                                           (3, 520, 1001, False)])
def test_latent_tail_writes_only_its_output(device, M, d, D, inplace):
    _say(f"guard latent_moe_tail M={M} d={d} D={D} inplace={inplace}")
    L, gamma, w_up, S = synth.tail_inputs(M, seed=70 + M, d=d, D=D)
    ws = GuardedWs(sg.sg_workspace_bytes(sg.SG_OP_LATENT_TAIL, M, D, d), device)
    if inplace:
        out = Guarded(M, D, device, init=dev(S, device))
        shared = out.view
    else:
        out = Guarded(M, D, device)
        shared = dev(S, device)
    sg.latent_moe_tail(dev(L, device), dev(gamma, device), dev(w_up, device), shared, out=out.view,
                       workspace=ws.view)
    torch.cuda.synchronize()
    out.check("tail output")
    ws.check("tail workspace")
    assert_close(out.bits(), oracle.latent_tail(L, gamma, 1e-6, w_up, S)[0], "guarded tail")


# ---- alternating shapes in one graph --------------------------------------------------

ALT_M = [1, 64, 4, 17, 256, 1, 13]


def test_alternating_shapes_in_one_graph(device):
    """Projection, Q/K/V/G alone and the tail at M = 1, 64, 4, 17, 256, 1, 13 in
    one graph over shared activations and one workspace per entry point,
    replayed three times; each replay must equal the eager sequence bit for
    bit."""
    K, nq = synth.HIDDEN, synth.N_QKVG
    mmax = max(ALT_M)
    x_all, packed, w_b = synth.overlap_inputs(mmax, seed=4321)
    L_all, gamma, w_up, S_all = synth.tail_inputs(mmax, seed=4322)
    xd, pd, wbd = dev(x_all, device), dev(packed, device), dev(w_b, device)
    Ld, gd, wud, Sd = (dev(a, device) for a in (L_all, gamma, w_up, S_all))
    ws_main = torch.zeros(max(sg.sg_kda_workspace_bytes(0, M, K, nq, 136) for M in ALT_M) + 256,
                          dtype=torch.uint8, device=device)
    ws_aux = torch.zeros(max(sg.sg_kda_workspace_bytes(1, M, K, nq, 136) for M in ALT_M) + 256,
                         dtype=torch.uint8, device=device)
    ws_q = torch.zeros(max(sg.sg_workspace_bytes(sg.SG_OP_GEMM, M, nq, K) for M in ALT_M) + 256,
                       dtype=torch.uint8, device=device)
    ws_t = torch.zeros(max(sg.sg_workspace_bytes(sg.SG_OP_LATENT_TAIL, M, synth.D_HIDDEN,
                                                 synth.D_LATENT) for M in ALT_M) + 256,
                       dtype=torch.uint8, device=device)

    def outs():
        return [(torch.empty((M, nq), dtype=torch.bfloat16, device=device),
                 torch.empty((M, synth.N_B), dtype=torch.bfloat16, device=device),
                 torch.empty((M, 8), dtype=torch.bfloat16, device=device),
                 torch.empty((M, nq), dtype=torch.bfloat16, device=device),
                 torch.empty((M, synth.D_HIDDEN), dtype=torch.bfloat16, device=device))
                for M in ALT_M]

    def run(o):
        for M, (q, g1, beta, q2, t) in zip(ALT_M, o):
            sg.kda_projection_overlap(xd[:M], pd, wbd, qkvg=q, g1=g1, beta=beta, ws_main=ws_main,
                                      ws_aux=ws_aux)
            sg.kda_qkvg_proj(xd[:M], pd[:nq], out=q2, workspace=ws_q)
            sg.latent_moe_tail(Ld[:M], gd, wud, Sd[:M], out=t, workspace=ws_t)

    eager = outs()
    run(eager)
    torch.cuda.synchronize()
    got = outs()
    side = torch.cuda.Stream(device)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            run(got)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        for group in got:
            for t in group:
                t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.ones(4096, device=device).sum()
        torch.cuda.synchronize()
        for M, a_grp, e_grp in zip(ALT_M, got, eager):
            for a, e in zip(a_grp, e_grp):
                assert torch.equal(a.view(torch.int16), e.view(torch.int16)), f"replay {rep} M={M}"
        del junk
    # the eager sequence itself against the oracle at two of its shapes
    for M in (4, 17):
        i = ALT_M.index(M)
        o = oracle.projection_overlap(x_all[:M], packed, w_b)
        assert_close(host(eager[i][0]), o["qkvg_exact"], f"alternating qkvg M={M}")
        assert_close(host(eager[i][1]), o["g1_exact"], f"alternating g1 M={M}")
        ex, _ = oracle.latent_tail(L_all[:M], gamma, 1e-6, w_up, S_all[:M])
        assert_close(host(eager[i][4]), ex, f"alternating tail M={M}")
