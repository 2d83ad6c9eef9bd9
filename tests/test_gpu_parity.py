"""GPU parity: every entry point of libskinny_gemm against the CPU oracle.

All calls go through the Python binding into the C ABI.  Inputs come from the
seeded generators in ``synth``; expected values only from ``oracle``.
Outputs are pre-filled with NaN so that an element a kernel forgets to write
fails the check.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bf16_skinny_gemm_02_amd as sg
import oracle
import synth
from tests.gpu_util import assert_close, cosine, dev, host, nan_like

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# ---- skinny_gemm over every kind, with ragged shapes --------------------------------

GEMM_CASES = [
    # (M, N, K, residual)  -- GEMV_ROW / SPLITK / SMALLK, MFMA WAVESPLIT / TILE /
    # BLOCK, ragged N and K
    (1, 1030, 1000, False), (2, 1500, 2056, True), (3, 1024, 520, False), (4, 1100, 7168, True),
    (5, 77, 3000, False), (8, 300, 1000, True), (11, 2000, 264, False), (16, 1100, 4104, True),
    (16, 40, 8, False), (4, 64, 136, True), (1, 5, 248, False), (7, 9, 256, True),
    (17, 300, 1000, False), (31, 100, 2056, True), (33, 520, 264, False), (64, 1024, 1000, True),
    (100, 77, 4104, False), (256, 300, 520, True), (255, 129, 96, False), (48, 3000, 40, True),
    (16, 1, 7168, False), (20, 1, 64, True), (3, 7, 0, True),
    (6, 5200, 1000, True), (13, 7170, 2056, False), (20, 9000, 512, True), (2, 4100, 7176, False),
    (130, 1000, 2056, True), (200, 4100, 520, False), (65, 7168, 2048, True), (129, 64, 1032, False),
    (12, 6000, 1032, True), (9, 8190, 264, False),
    # one workgroup per CU of 17..32 rows (two 16-row fragments): a ragged
    # first fragment in the last tile, and whole 32-row tiles
    (3, 5124, 2048, True), (16, 8192, 1032, False),
    # long K: GEMV ranges at their full depth, split wave-split partials, 52-way tile and
    # block splits (the reduction's loop over many partials)
    (1, 300, 65536, False), (8, 500, 32768, True), (64, 256, 16384, True), (200, 128, 16392, False),
    (16, 2000, 40000, True),
    # 17 <= M <= 32 with wide N (64-row tiles, K split, reduction)
    (24, 7168, 2048, True), (32, 8000, 1000, False), (17, 6200, 4104, True),
]


@pytest.mark.parametrize("M,N,K,res", GEMM_CASES)
def test_skinny_gemm_matches_oracle(device, M, N, K, res):
    _say(f"skinny_gemm M={M} N={N} K={K} res={res} cfg={sg.sg_select(M, N, K, res)}")
    A, W, R = synth.gemm_inputs(M, N, K, seed=9000 + M * 7 + N + K, residual=res)
    out = nan_like((M, N), device)
    sg.skinny_gemm(dev(A, device), dev(W, device), dev(R, device) if res else None, out=out)
    torch.cuda.synchronize()
    ex, _ = oracle.gemm(A, W, R)
    assert_close(host(out), ex, f"skinny_gemm {M}x{N}x{K}")


def test_skinny_gemm_strided_activation_and_inplace_residual(device):
    M, N, K = 6, 2048, 1024
    A, W, R = synth.gemm_inputs(M, N, K, seed=77, residual=True)
    big = torch.zeros((M, K + 64), dtype=torch.bfloat16, device=device)
    big[:, 8:8 + K] = dev(A, device)
    a_view = big[:, 8:8 + K]              # row stride K + 64, 16-byte aligned start
    c = dev(R, device).clone()            # output aliases the residual
    sg.skinny_gemm(a_view, dev(W, device), c, out=c)
    torch.cuda.synchronize()
    ex, _ = oracle.gemm(A, W, R)
    assert_close(host(c), ex, "strided + in-place")


def test_skinny_gemm_explicit_config(device):
    M, N, K = 4, 1024, 2048
    A, W, _ = synth.gemm_inputs(M, N, K, seed=78)
    cfg = sg.sg_select(M, N, K)
    out = sg.skinny_gemm(dev(A, device), dev(W, device), cfg=cfg)
    out2 = sg.skinny_gemm(dev(A, device), dev(W, device))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


# ---- the KDA Q/K/V/G projection at full size ----------------------------------------

QKVG_M = [1, 2, 3, 4, 8, 16, 17, 32, 64]


@pytest.mark.parametrize("M", QKVG_M)
def test_qkvg_full_size(device, M):
    cfg = sg.sg_select(M, synth.N_QKVG, synth.HIDDEN)
    _say(f"kda_qkvg_proj M={M} cfg={cfg}")
    x, w = synth.qkvg_inputs(M)
    out = nan_like((M, synth.N_QKVG), device)
    sg.kda_qkvg_proj(dev(x, device), dev(w, device), out=out)
    torch.cuda.synchronize()
    ex, _ = oracle.qkvg(x, w)
    g = host(out)
    assert_close(g, ex, f"qkvg M={M}")
    assert cosine(g, ex) > 0.9999


@pytest.mark.parametrize("M", [1, 3, 16, 17, 64, 100, 256])
def test_qkvg_lattice_bitwise(device, M):
    """On the integer lattice fp32 accumulation is exact in any order, so the
    GPU must equal the oracle bit for bit."""
    K, N = synth.HIDDEN, synth.N_QKVG
    x = synth.lattice_activation((M, K), seed=300 + M)
    w = synth.lattice_weight((N, K), seed=400 + M)
    out = nan_like((M, N), device)
    sg.kda_qkvg_proj(dev(x, device), dev(w, device), out=out)
    torch.cuda.synchronize()
    _, bits = oracle.qkvg(x, w)
    assert np.array_equal(host(out), bits)


def test_qkvg_repeat_is_deterministic(device):
    x, w = synth.qkvg_inputs(5)
    xd, wd = dev(x, device), dev(w, device)
    a = sg.kda_qkvg_proj(xd, wd)
    b = sg.kda_qkvg_proj(xd, wd)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---- F_A/beta -> F_B ------------------------------------------------------------------

@pytest.mark.parametrize("M", [1, 2, 4, 8, 16, 32, 64, 128])
@pytest.mark.parametrize("n_ab", [136, 140, 144])
def test_fab_fb_matches_oracle(device, M, n_ab):
    cfg = sg.sg_kda_select(sg.SG_KDA_FAB_ALONE, M, synth.HIDDEN, 0, n_ab)
    _say(f"kda_fab_fb_proj M={M} n_ab={n_ab} cfg={cfg}")
    x, w_ab, w_b = synth.fab_fb_inputs(M, n_ab=n_ab)
    beta = nan_like((M, n_ab - 128), device)
    g1 = nan_like((M, synth.N_B), device)
    g1, beta, f_a = sg.kda_fab_fb_proj(dev(x, device), dev(w_ab, device), dev(w_b, device),
                                       want_f_a=True, beta=beta, g1=g1)
    torch.cuda.synchronize()
    o = oracle.fab_fb(x, w_ab, w_b)
    assert_close(host(f_a), o["p_exact"][:, :128], "f_a")
    assert_close(host(beta), o["beta_exact"], "beta")
    assert_close(host(g1), o["g1_exact"], "g1")


@pytest.mark.parametrize("M", [1, 8, 32])
def test_fab_fb_lattice_bitwise(device, M):
    K, n_ab, rank, n_b = synth.HIDDEN, 136, 128, 1024
    x = synth.lattice_activation((M, K), seed=500 + M)
    w_ab = synth.lattice_weight((n_ab, K), seed=600 + M)
    w_b = synth.lattice_weight((n_b, rank), seed=700 + M)
    g1, beta, f_a = sg.kda_fab_fb_proj(dev(x, device), dev(w_ab, device), dev(w_b, device),
                                       want_f_a=True)
    torch.cuda.synchronize()
    o = oracle.fab_fb(x, w_ab, w_b)
    assert np.array_equal(host(f_a), o["f_a"])
    assert np.array_equal(host(beta), o["beta"])
    assert np.array_equal(host(g1), o["g1_bits"])


@pytest.mark.parametrize("M,K", [(1, 16384), (2, 16384), (3, 12288)])
def test_fab_fb_long_k(device, M, K):
    """Long K: the standalone F_A/beta rows keep at most 8 K-ranges, one
    batch of partials for the F_B stage, so each range is long (up to 2048
    columns here).  (More splits than one batch are covered through the
    projection's F_A/beta range below.)"""
    cfg = sg.sg_kda_select(sg.SG_KDA_FAB_ALONE, M, K, 4096, 136)
    _say(f"kda_fab_fb_proj long K M={M} K={K} cfg={cfg}")
    assert cfg["k_split"] == 8
    x, w_ab, w_b = synth.fab_fb_inputs(M, seed=77 + M, K=K)
    g1, beta, f_a = sg.kda_fab_fb_proj(dev(x, device), dev(w_ab, device), dev(w_b, device),
                                       want_f_a=True)
    torch.cuda.synchronize()
    o = oracle.fab_fb(x, w_ab, w_b)
    assert_close(host(f_a), o["p_exact"][:, :128], "f_a")
    assert_close(host(beta), o["beta_exact"], "beta")
    assert_close(host(g1), o["g1_exact"], "g1")


@pytest.mark.parametrize("M", [3, 12])
def test_projection_many_splits(device, M):
    """A small Q/K/V/G range (256 rows): the paired tiles split K 28 ways, so
    the F_B launch sums 28 F_A/beta partials (batches, then its loop) and its
    reduction role 28 Q/K/V/G partials (straight-line batches, then a loop);
    both schedules against each other and the oracle."""
    K, nq = synth.HIDDEN, 256
    cq = sg.sg_kda_select(sg.SG_KDA_QKVG, M, K, nq, 136)
    _say(f"kda_projection_overlap many splits M={M} n_qkvg={nq} cfg={cq}")
    assert cq["k_split"] > 16
    x, packed, w_b = synth.overlap_inputs(M, seed=88 + M, n_qkvg=nq)
    xd, pd, wbd = dev(x, device), dev(packed, device), dev(w_b, device)
    aux = torch.cuda.Stream(device)
    fork, join = sg.HipEvent(), sg.HipEvent()
    q_s, g1_s, b_s = sg.kda_projection_overlap(xd, pd, wbd, n_qkvg=nq)
    q_c, g1_c, b_c = sg.kda_projection_overlap(xd, pd, wbd, n_qkvg=nq, aux_stream=aux, fork=fork,
                                               join=join)
    torch.cuda.synchronize()
    for a, b in ((q_c, q_s), (g1_c, g1_s), (b_c, b_s)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    o = oracle.projection_overlap(x, packed, w_b, n_qkvg=nq)
    assert_close(host(q_s), o["qkvg_exact"], "qkvg")
    assert_close(host(g1_s), o["g1_exact"], "g1")
    assert_close(host(b_s), o["beta_exact"], "beta")


# ---- the concurrent projection ------------------------------------------------------------

@pytest.mark.parametrize("M", [1, 4, 16, 17, 32, 48, 64])
def test_overlap_matches_sequential_and_oracle(device, M):
    _say(f"kda_projection_overlap M={M}")
    x, packed, w_b = synth.overlap_inputs(M)
    xd, pd, wbd = dev(x, device), dev(packed, device), dev(w_b, device)
    aux = torch.cuda.Stream(device)
    fork, join = sg.HipEvent(), sg.HipEvent()
    q_c, g1_c, b_c = sg.kda_projection_overlap(xd, pd, wbd, aux_stream=aux, fork=fork, join=join)
    q_s, g1_s, b_s = sg.kda_projection_overlap(xd, pd, wbd)
    torch.cuda.synchronize()
    for a, b in ((q_c, q_s), (g1_c, g1_s), (b_c, b_s)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    o = oracle.projection_overlap(x, packed, w_b)
    assert_close(host(q_c), o["qkvg_exact"], "qkvg")
    assert_close(host(g1_c), o["g1_exact"], "g1")
    assert_close(host(b_c), o["beta_exact"], "beta")


@pytest.mark.parametrize("concurrent", [True, False])
@pytest.mark.parametrize("M", [1, 4, 16, 32])
def test_overlap_graph_replay(device, M, concurrent):
    """Capture the KDA projection (the two-stream fork/join schedule, or the
    single-stream one the closed gate picks) in a graph, replay it several
    times with eager work in between, and compare every replay bit for bit
    with the eager single-stream result."""
    _say(f"kda_projection_overlap graph M={M} concurrent={concurrent}")
    x, packed, w_b = synth.overlap_inputs(M)
    xd, pd, wbd = dev(x, device), dev(packed, device), dev(w_b, device)
    aux = torch.cuda.Stream(device)
    fork, join = sg.HipEvent(), sg.HipEvent()
    q_e, g1_e, b_e = sg.kda_projection_overlap(xd, pd, wbd)
    q = torch.empty_like(q_e)
    g1 = torch.empty_like(g1_e)
    beta = torch.empty_like(b_e)
    ws_aux = torch.zeros(max(sg.sg_kda_workspace_bytes(1, M, synth.HIDDEN, 4096, 136), 256),
                         dtype=torch.uint8, device=device)
    ws_main = torch.zeros(max(sg.sg_kda_workspace_bytes(0, M, synth.HIDDEN, 4096, 136), 256),
                          dtype=torch.uint8, device=device)
    kw = dict(aux_stream=aux, fork=fork, join=join) if concurrent else {}
    side = torch.cuda.Stream(device)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            sg.kda_projection_overlap(xd, pd, wbd, qkvg=q, g1=g1, beta=beta, ws_aux=ws_aux,
                                      ws_main=ws_main, **kw)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        for t in (q, g1, beta):
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        junk = sg.kda_qkvg_proj(xd, pd[:4096])  # eager work between replays
        torch.cuda.synchronize()
        for a, b in ((q, q_e), (g1, g1_e), (beta, b_e)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}"
        del junk


def _replay_check(device, capture_fn, outs, eager, reps=4):
    """Capture capture_fn() on a side stream, replay it `reps` times with
    eager work and synchronisations in between, and compare every replay
    with the eager outputs bit for bit."""
    side = torch.cuda.Stream(device)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            capture_fn()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(reps):
        for t in outs:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.ones(1024, device=device).sum()  # eager work between replays
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}"
        del junk


@pytest.mark.parametrize("M", [1, 8, 17, 64, 100])
def test_qkvg_graph_replay(device, M):
    """The single-launch (M <= 16), split-K + reduction (M > 16) and block
    (M > 64) Q/K/V/G paths inside a captured graph."""
    _say(f"kda_qkvg_proj graph M={M}")
    x, w = synth.qkvg_inputs(M)
    xd, wd = dev(x, device), dev(w, device)
    eager = sg.kda_qkvg_proj(xd, wd)
    out = torch.empty_like(eager)
    ws = torch.empty(max(sg.sg_workspace_bytes(sg.SG_OP_GEMM, M, synth.N_QKVG, synth.HIDDEN), 256),
                     dtype=torch.uint8, device=device)
    _replay_check(device, lambda: sg.kda_qkvg_proj(xd, wd, out=out, workspace=ws), [out], [eager])


@pytest.mark.parametrize("M", [1, 4, 16, 64])
def test_latent_tail_graph_replay(device, M):
    """The tail's GEMV fold (M = 1), wave-split fold (M = 4) and norm kernel +
    GEMM (+ reduction) paths inside a captured graph."""
    _say(f"latent_moe_tail graph M={M}")
    L, gamma, w_up, S = synth.tail_inputs(M)
    args = [dev(a, device) for a in (L, gamma, w_up, S)]
    eager = sg.latent_moe_tail(*args)
    out = torch.empty_like(eager)
    ws = torch.empty(max(sg.sg_workspace_bytes(sg.SG_OP_LATENT_TAIL, M, synth.D_HIDDEN,
                                               synth.D_LATENT), 256),
                     dtype=torch.uint8, device=device)
    _replay_check(device, lambda: sg.latent_moe_tail(*args, out=out, workspace=ws), [out], [eager])


@pytest.mark.parametrize("M", [1, 3, 8, 16, 17, 64, 100])
def test_sequential_projection_equals_separate_calls(device, M):
    """The sequential KDA projection (Q/K/V/G and F_A/beta as two segments of
    one launch, then F_B with the Q/K/V/G split-K reduction) against
    kda_qkvg_proj + kda_fab_fb_proj: bit for bit the same outputs wherever
    sg_kda_select gives the same configurations as the standalone calls
    (always for 64 < M, where the projection takes the table's block tiles;
    at M = 1 when the standalone F_A/beta rows also take 7 K-ranges); at
    2 <= M <= 64 the projection pairs its ranges in 128-row tiles with another
    K split, so the sums round in another order, and wherever the
    configurations differ both must meet the oracle's tolerance instead."""
    _say(f"sequential projection vs separate calls M={M}")
    K = synth.HIDDEN
    x, packed, w_b = synth.overlap_inputs(M)
    xd, pd, wbd = dev(x, device), dev(packed, device), dev(w_b, device)
    q_s, g1_s, b_s = sg.kda_projection_overlap(xd, pd, wbd)
    q = sg.kda_qkvg_proj(xd, pd[:4096])
    g1, beta = sg.kda_fab_fb_proj(xd, pd[4096:], wbd)
    torch.cuda.synchronize()
    same = (sg.sg_kda_select(sg.SG_KDA_QKVG, M, K, 4096, 136) == sg.sg_select(M, 4096, K) and
            sg.sg_kda_select(sg.SG_KDA_FAB, M, K, 4096, 136) ==
            sg.sg_kda_select(sg.SG_KDA_FAB_ALONE, M, K, 4096, 136))
    if M > 64:
        assert same
    if 2 <= M <= 64:
        assert not same
    if same:
        for a, b in ((q_s, q), (g1_s, g1), (b_s, beta)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    else:
        o = oracle.projection_overlap(x, packed, w_b)
        for a, b, ex, name in ((q_s, q, o["qkvg_exact"], "qkvg"), (g1_s, g1, o["g1_exact"], "g1"),
                               (b_s, beta, o["beta_exact"], "beta")):
            assert_close(host(a), ex, name + " (projection)")
            assert_close(host(b), ex, name + " (separate calls)")


@pytest.mark.parametrize("M", [2, 7, 12, 16, 17, 48, 64])
def test_projection_lattice_bitwise(device, M):
    """Integer-lattice inputs make every partial sum exact in fp32, so the
    projection (including the paired 128-row tiles at 2 <= M <= 64) must equal
    the oracle bit for bit whatever its split and summation order."""
    _say(f"projection lattice M={M} q={sg.sg_kda_select(0, M, synth.HIDDEN, 4096, 136)}")
    K = synth.HIDDEN
    x = synth.lattice_activation((M, K), seed=800 + M)
    packed = synth.lattice_weight((4096 + 136, K), seed=900 + M)
    w_b = synth.lattice_weight((1024, 128), seed=1000 + M)
    q, g1, beta = sg.kda_projection_overlap(dev(x, device), dev(packed, device), dev(w_b, device))
    torch.cuda.synchronize()
    o = oracle.projection_overlap(x, packed, w_b)
    assert np.array_equal(host(q), o["qkvg_bits"])
    assert np.array_equal(host(beta), o["beta"])
    assert np.array_equal(host(g1), o["g1_bits"])


def test_packed_projection_equals_split(device):
    """The packed [W_qkvg; W_ab] GEMM (the sequential fallback's first step)
    reproduces the Q/K/V/G columns bit for bit and F_A/beta within tolerance."""
    M = 4
    x, packed, w_b = synth.overlap_inputs(M)
    xd, pd = dev(x, device), dev(packed, device)
    full = sg.skinny_gemm(xd, pd)
    q = sg.kda_qkvg_proj(xd, pd[:4096])
    torch.cuda.synchronize()
    assert torch.equal(full[:, :4096].view(torch.int16), q.view(torch.int16))
    ex, _ = oracle.gemm(x, packed)
    assert_close(host(full), ex, "packed")


# ---- latent-MoE tail ----------------------------------------------------------------------

@pytest.mark.parametrize("M", [1, 2, 8, 13, 16, 17, 24, 32, 33, 64, 130, 256])
def test_latent_tail_full_size(device, M):
    cfg = sg.sg_select(M, synth.D_HIDDEN, synth.D_LATENT)
    _say(f"latent_moe_tail M={M} cfg={cfg}")
    L, gamma, w_up, S = synth.tail_inputs(M)
    out = nan_like((M, synth.D_HIDDEN), device)
    sg.latent_moe_tail(dev(L, device), dev(gamma, device), dev(w_up, device), dev(S, device),
                       eps=1e-6, out=out)
    torch.cuda.synchronize()
    ex, _ = oracle.latent_tail(L, gamma, 1e-6, w_up, S)
    g = host(out)
    assert_close(g, ex, f"tail M={M}")
    assert cosine(g, ex) > 0.9999


@pytest.mark.parametrize("M", [3, 20])
def test_latent_tail_no_shared_and_inplace(device, M):
    d, D = 2048, 7168
    L, gamma, w_up, S = synth.tail_inputs(M, seed=4242 + M)
    Ld, gd, wd = dev(L, device), dev(gamma, device), dev(w_up, device)
    out = sg.latent_moe_tail(Ld, gd, wd, None, eps=1e-5)
    inplace = dev(S, device).clone()
    sg.latent_moe_tail(Ld, gd, wd, inplace, eps=1e-5, out=inplace)
    torch.cuda.synchronize()
    ex, _ = oracle.latent_tail(L, gamma, 1e-5, w_up, None)
    assert_close(host(out), ex, "tail without shared")
    ex_s, _ = oracle.latent_tail(L, gamma, 1e-5, w_up, S)
    assert_close(host(inplace), ex_s, "tail in place")


@pytest.mark.parametrize("M", [2, 40])
def test_latent_tail_zero_weights_is_shared(device, M):
    L, gamma, w_up, S = synth.tail_inputs(M, seed=99)
    zero = torch.zeros((synth.D_HIDDEN, synth.D_LATENT), dtype=torch.bfloat16, device=device)
    out = sg.latent_moe_tail(dev(L, device), dev(gamma, device), zero, dev(S, device))
    torch.cuda.synchronize()
    assert np.array_equal(host(out), S)


@pytest.mark.parametrize("M,d,D", [(5, 264, 900), (24, 520, 100), (2, 128, 64),
                                   (3, 1000, 5200), (11, 4104, 6000), (16, 2048, 5136),
                                   (4, 2048, 1024), (7, 1032, 3000), (12, 2048, 2000),
                                   (16, 1024, 4096), (20, 2048, 6400), (29, 1032, 8192)])
def test_latent_tail_other_shapes(device, M, d, D):
    """Shapes that take the split-K, small-latent and folded-RMSNorm paths of
    the tail: the GEMV fold (M = 1), the wave-split fold (ragged latent, a
    K split, every activation-row group), and the separate norm kernel."""
    _say(f"latent_moe_tail M={M} d={d} D={D} cfg={sg.sg_select(M, D, d)}")
    L, gamma, w_up, S = synth.tail_inputs(M, seed=123 + M, d=d, D=D)
    out = nan_like((M, D), device)
    sg.latent_moe_tail(dev(L, device), dev(gamma, device), dev(w_up, device), dev(S, device),
                       out=out)
    torch.cuda.synchronize()
    ex, _ = oracle.latent_tail(L, gamma, 1e-6, w_up, S)
    assert_close(host(out), ex, f"tail {M}x{d}->{D}")


@pytest.mark.parametrize("M,d,D", [(17, 2048, 7168), (32, 2048, 7168), (64, 2048, 7168),
                                   (24, 4104, 640), (40, 520, 1000)])
def test_latent_tail_split_k_reused_workspace(device, M, d, D):
    """The tail's norm launch, split-K tile GEMM and fixed-order reduction
    share one workspace (normalised latent, then partials).  One workspace,
    first filled with 0xFF bytes, serves three calls on different inputs:
    every call must match the oracle, so nothing of another call (or of the
    fill) can leak into a result."""
    cfg = sg.sg_select(M, D, d)
    _say(f"latent_moe_tail split-K M={M} d={d} D={D} cfg={cfg}")
    assert cfg["kind"] == sg.SG_KIND_MFMA_TILE and cfg["k_split"] > 1
    ws = torch.full((sg.sg_workspace_bytes(sg.SG_OP_LATENT_TAIL, M, D, d),), 255,
                    dtype=torch.uint8, device=device)
    for seed in (7, 8, 9):
        L, gamma, w_up, S = synth.tail_inputs(M, seed=seed * 1000 + M, d=d, D=D)
        out = nan_like((M, D), device)
        sg.latent_moe_tail(dev(L, device), dev(gamma, device), dev(w_up, device), dev(S, device),
                           out=out, workspace=ws)
        torch.cuda.synchronize()
        ex, _ = oracle.latent_tail(L, gamma, 1e-6, w_up, S)
        assert_close(host(out), ex, f"split-K tail {M}x{d}->{D} seed {seed}")


def test_empty_problems_are_noops(device):
    x = torch.zeros((0, 7168), dtype=torch.bfloat16, device=device)
    w = torch.zeros((4096, 7168), dtype=torch.bfloat16, device=device)
    assert sg.kda_qkvg_proj(x, w).shape == (0, 4096)
