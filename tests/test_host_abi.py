"""Host-side tests of libskinny_gemm (no GPU needed).

* the shared library loads and exports every function include/skinny_gemm.h
  declares;
* the configuration table and the overlap gate agree field by field with the
  independent selection oracle, over an exhaustive grid of shapes;
* every entry point rejects invalid arguments with the documented status, and
  returns before touching the GPU (validation happens before any HIP call).
"""
from __future__ import annotations

import ctypes
import itertools
import re
from pathlib import Path

import pytest

from bf16_skinny_gemm_02_amd import _lib
from oracle import selection

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "skinny_gemm.h"


@pytest.fixture(scope="module")
def lib():
    if not _lib.LIB_PATH.exists():
        pytest.fail(f"{_lib.LIB_PATH} not built: run `python -m bf16_skinny_gemm_02_amd.build`")
    return _lib.load()


def _declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_expected_entry_points():
    names = _declared_functions()
    assert set(names) == set(_lib.EXPORTED_SYMBOLS), names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_strerror_and_version(lib):
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert lib.sg_strerror(st)
    assert re.fullmatch(rb"\d+\.\d+\.\d+", lib.sg_version())


# ---- configuration table ------------------------------------------------------------

SHAPES = [(4096, 7168), (136, 7168), (140, 7168), (144, 7168), (1024, 128), (7168, 2048),
          (4232, 7168), (1, 8), (3, 16), (1000, 1000), (300, 264), (17, 0), (0, 64), (5, 256),
          (5, 264), (1023, 4096), (1024, 4096), (2048, 520), (3072, 6144), (100, 2)]


def _c_select(lib, M, N, K, res):
    cfg = _lib.SgConfig()
    st = lib.sg_select(M, N, K, res, ctypes.byref(cfg))
    return st, cfg.as_dict()


def test_select_matches_oracle_exhaustive(lib):
    checked = 0
    for (N, K), M, res in itertools.product(SHAPES, range(-1, 301), (0, 1)):
        st_c, cfg_c = _c_select(lib, M, N, K, res)
        st_o, cfg_o = selection.select(M, N, K, bool(res))
        assert st_c == st_o, (M, N, K)
        if st_o == selection.OK:
            assert cfg_c == cfg_o, (M, N, K, cfg_c, cfg_o)
        checked += 1
    assert checked > 10000


def test_select_matches_oracle_random(lib):
    import random
    rnd = random.Random(1234)
    for _ in range(20000):
        M = rnd.randint(-2, 300)
        N = rnd.choice([rnd.randint(-2, 40), rnd.randint(0, 20000)])
        K = rnd.choice([rnd.randint(-2, 600), 8 * rnd.randint(0, 2000)])
        res = rnd.randint(0, 1)
        st_c, cfg_c = _c_select(lib, M, N, K, res)
        st_o, cfg_o = selection.select(M, N, K, bool(res))
        assert st_c == st_o, (M, N, K)
        if st_o == selection.OK:
            assert cfg_c == cfg_o, (M, N, K)


def test_select_null_out(lib):
    assert lib.sg_select(1, 1, 8, 0, None) == _lib.SG_ERR_INVALID_ARG


def _kind_for(M):
    if M == 1:
        return selection.GEMV_ROW
    if M <= 16:
        return selection.MFMA_WAVESPLIT
    return selection.MFMA_TILE if M <= 64 else selection.MFMA_BLOCK


def test_kind_follows_m_boundaries():
    for M in range(1, 257):
        st, cfg = selection.select(M, 4096, 7168)
        assert st == selection.OK
        assert cfg["kind"] == _kind_for(M), M
    # Past 320 tiles of 16 rows, M <= 16 stays on the wave-split tile with
    # one workgroup per CU of up to 32 rows (two fragments): 7168 rows are
    # 256 workgroups of 28 (the rule; at K = 2048, the tail's shape, the
    # measured table decides instead).  Wider N moves to the
    # shared-activation tile (32 rows).
    for M in (2, 8, 12, 16):
        cfg = selection.select(M, 7168, 2056)[1]
        assert cfg["kind"] == selection.MFMA_WAVESPLIT
        assert (cfg["rows"], cfg["k_unroll"], cfg["grid"]) == (28, 3, 256)
    assert selection.select(8, 5200, 2048)[1]["rows"] == 24
    assert selection.select(8, 5120, 2048)[1]["rows"] == 16
    assert selection.select(8, 8192, 2048)[1]["rows"] == 32
    assert selection.select(8, 9000, 2048)[1]["kind"] == selection.MFMA_TILE
    assert selection.select(12, 9000, 2048)[1]["kind"] == selection.MFMA_TILE
    assert selection.select(12, 9000, 2048)[1]["rows"] == 32
    # M = 1 takes seven rows per wave when a whole row fits four 512-wide
    # steps (the tail's 7168 x 2048: exactly 256 workgroups), four rows when
    # it fits seven.
    assert selection.select(1, 7168, 2048)[1]["rows"] == 7
    assert selection.select(1, 7168, 2048)[1]["grid"] == 256
    assert selection.select(1, 7168, 3584)[1]["rows"] == 4
    assert selection.select(1, 4096, 7168)[1]["rows"] == 1
    assert selection.select(257, 4096, 7168)[0] == selection.UNSUPPORTED
    assert selection.select(0, 4096, 7168)[1]["kind"] == selection.NONE


KDA_SHAPES = [(7168, 4096, 136), (7168, 4096, 140), (7168, 4096, 144), (2048, 1024, 136),
              (128, 512, 136), (7168, 0, 136), (264, 64, 16), (7168, 4096, 0), (1000, 300, 40),
              (7168, 40000, 136), (8, 8, 8), (520, 4096, 260), (131072, 4096, 136),
              (16384, 256, 136)]


def _c_kda_select(lib, which, M, K, nq, nab):
    cfg = _lib.SgConfig()
    st = lib.sg_kda_select(which, M, K, nq, nab, ctypes.byref(cfg))
    return st, cfg.as_dict()


def test_kda_select_matches_oracle(lib):
    checked = 0
    for (K, nq, nab), M, which in itertools.product(KDA_SHAPES, range(-1, 260), (-1, 0, 1, 2, 3)):
        st_c, cfg_c = _c_kda_select(lib, which, M, K, nq, nab)
        st_o, cfg_o = selection.kda_select(which, M, K, nq, nab)
        assert st_c == st_o, (which, M, K, nq, nab)
        if st_o == selection.OK:
            assert cfg_c == cfg_o, (which, M, K, nq, nab, cfg_c, cfg_o)
        checked += 1
        for w in (0, 1):
            if which == w:
                assert lib.sg_kda_workspace_bytes(w, M, K, nq, nab) == \
                    selection.kda_workspace_bytes(w, M, K, nq, nab), (w, M, K, nq, nab)
    assert checked > 10000
    assert lib.sg_kda_select(0, 1, 8, 8, 8, None) == _lib.SG_ERR_INVALID_ARG


def test_fab_k_ranges_fit_one_batch():
    """The F_A/beta rows keep at most 8 K-ranges (one batch of partials for the
    F_B stage) unless a GEMV wave could not hold its range: then as few as fit
    16 of its 512-wide steps."""
    for K in (2048, 7168, 16384, 65536, 131072, 262144):
        for M in (1, 2, 16, 64, 65, 256):
            st, f = selection.kda_select(2, M, K, 0, 136)
            assert st == selection.OK
            if f["kind"] in (selection.GEMV_SPLITK, selection.GEMV_ROW):
                steps = -(-(K // 8) // 64)
                per = -(-steps // f["k_split"])
                assert per <= 16 and (f["k_split"] <= 8 or per == 16), (M, K, f)
            else:
                assert f["k_split"] <= 8, (M, K, f)
            assert f["grid"] % f["k_split"] == 0


def test_kda_select_pairs_the_projection_tiles():
    # 2 <= M <= 64 at the KDA shapes: both ranges in 128-row tiles, one K split,
    # (32 + 2) * 7 = 238 workgroups: one round on 256 CUs.
    for M in (2, 3, 8, 12, 16, 17, 32, 48, 64):
        _, q = selection.kda_select(0, M, 7168, 4096, 136)
        _, f = selection.kda_select(1, M, 7168, 4096, 136)
        assert (q["rows"], q["waves"], q["k_split"], q["grid"]) == (128, 8, 7, 224)
        assert (f["rows"], f["waves"], f["k_split"], f["grid"]) == (128, 8, 7, 14)
        assert q["m_tile"] == (4 * -(-M // 4) if M <= 16 else 16 * -(-M // 16))
        # the standalone calls keep the table's own kernels (the 128-row
        # tile too where the measured table picked it)
        assert selection.select(M, 4096, 7168)[1]["rows"] in (16, 64, 128)
        assert selection.kda_select(2, M, 7168, 4096, 136)[1]["rows"] in (16, 64, 128)
    for M in (1, 65, 256):
        assert selection.kda_select(0, M, 7168, 4096, 136)[1] == selection.select(M, 4096, 7168)[1]


def test_overlap_gate_matches_oracle(lib):
    # Measured on MI355X: the two-stream schedule never won, so the gate is
    # closed at every M (the setting, not the rule, is what is pinned here).
    assert lib.sg_overlap_max_tokens() == selection.OVERLAP_MAX_TOKENS == 0
    assert not any(lib.sg_overlap_gate(M, 1, 1, 1, 1) for M in range(0, 300))
    for M, c, a, e, en in itertools.product(range(-1, 70), (0, 1), (0, 1), (0, 1), (0, 1)):
        assert bool(lib.sg_overlap_gate(M, c, a, e, en)) == selection.overlap_gate(M, c, a, e, en)


def test_workspace_bytes(lib):
    # QKVG for M <= 16 needs no workspace (one launch, no K split); the
    # tiles for M > 16 split K (the 64-row tile four ways at M = 32, the
    # measured table's 128-row tile eight ways at M = 64); F_A/beta always
    # keeps partials.
    assert lib.sg_workspace_bytes(_lib.SG_OP_GEMM, 1, 4096, 7168) == 0
    assert lib.sg_workspace_bytes(_lib.SG_OP_GEMM, 8, 4096, 7168) == 0
    assert lib.sg_workspace_bytes(_lib.SG_OP_GEMM, 32, 4096, 7168) == 4 * 32 * 4096 * 4
    assert lib.sg_workspace_bytes(_lib.SG_OP_GEMM, 64, 4096, 7168) == 8 * 64 * 4096 * 4
    # The standalone F_A/beta -> F_B call sizes its partials for the F_A/beta
    # configuration it runs alone, at most 8 K-ranges at the projection shape.
    for M in (1, 2, 4, 8, 16, 32, 64, 65, 200):
        st, cfg = selection.kda_select(2, M, 7168, 0, 136)
        assert st == selection.OK
        assert 1 <= cfg["k_split"] <= 8
        need = lib.sg_workspace_bytes(_lib.SG_OP_FAB_FB, M, 136, 7168)
        # the hand-off header of the one-launch entry point, then the partials
        assert need == 18432 + (cfg["k_split"] * M * 136 * 4 + 255) // 256 * 256
    assert lib.sg_workspace_bytes(_lib.SG_OP_GEMM, -1, 4, 8) == 0
    assert lib.sg_workspace_bytes(99, 4, 4, 8) == 0


# ---- argument validation (host only: every call returns before any HIP call) ----------

A16 = ctypes.c_void_p(0x10000)    # 16-byte aligned fake device addresses: never dereferenced
B16 = ctypes.c_void_p(0x20000)
C16 = ctypes.c_void_p(0x30000)
ODD = ctypes.c_void_p(0x10008)    # 8-byte aligned only
NUL = None


def _gemm(lib, A=A16, lda=64, W=B16, ldw=64, R=NUL, ldr=32, C=C16, ldc=32, M=4, N=32, K=64,
          cfg=None, ws=NUL, ws_bytes=0):
    return lib.skinny_gemm(A, lda, W, ldw, R, ldr, C, ldc, M, N, K, cfg, ws, ws_bytes, None)


def test_skinny_gemm_validation(lib):
    E = _lib
    assert _gemm(lib, M=-1) == E.SG_ERR_INVALID_ARG
    assert _gemm(lib, K=-8) == E.SG_ERR_INVALID_ARG
    assert _gemm(lib, K=60) == E.SG_ERR_UNSUPPORTED
    assert _gemm(lib, M=257) == E.SG_ERR_UNSUPPORTED
    assert _gemm(lib, A=NUL) == E.SG_ERR_INVALID_ARG
    assert _gemm(lib, W=NUL) == E.SG_ERR_INVALID_ARG
    assert _gemm(lib, C=NUL) == E.SG_ERR_INVALID_ARG
    assert _gemm(lib, lda=32) == E.SG_ERR_INVALID_ARG
    assert _gemm(lib, ldc=16) == E.SG_ERR_INVALID_ARG
    assert _gemm(lib, A=ODD) == E.SG_ERR_MISALIGNED
    assert _gemm(lib, W=ODD) == E.SG_ERR_MISALIGNED
    assert _gemm(lib, lda=68) == E.SG_ERR_MISALIGNED
    assert _gemm(lib, C=ctypes.c_void_p(0x30001)) == E.SG_ERR_MISALIGNED
    assert _gemm(lib, R=ctypes.c_void_p(0x40001)) == E.SG_ERR_MISALIGNED
    # a config the kernels cannot run (no 1-row MFMA tile), and one they can
    # whose K split needs a workspace
    bad = _lib.SgConfig(kind=4, m_tile=16, rows=1, waves=4, k_split=1, k_unroll=8, grid=2)
    assert _gemm(lib, cfg=ctypes.byref(bad)) == E.SG_ERR_UNSUPPORTED
    alt = _lib.SgConfig(kind=5, m_tile=4, rows=16, waves=4, k_split=2, k_unroll=3, grid=4,
                        nt_weights=1)
    assert lib.sg_config_supported(ctypes.byref(alt), 4, 32, 64) == E.SG_OK
    assert _gemm(lib, cfg=ctypes.byref(alt)) == E.SG_ERR_WORKSPACE
    need = lib.sg_config_workspace_bytes(ctypes.byref(alt), 4, 32)
    assert need == 2 * 4 * 32 * 4 + 0  # one 256-byte rounded plane pair: 1024 bytes
    assert _gemm(lib, cfg=ctypes.byref(alt), ws=ctypes.c_void_p(0x50000), ws_bytes=need - 1) == \
        E.SG_ERR_WORKSPACE
    # a split-K shape without workspace
    st, cfg = selection.select(4, 32, 4096)
    assert cfg["k_split"] > 1
    assert _gemm(lib, lda=4096, ldw=4096, K=4096) == E.SG_ERR_WORKSPACE
    need = lib.sg_workspace_bytes(_lib.SG_OP_GEMM, 4, 32, 4096)
    assert _gemm(lib, lda=4096, ldw=4096, K=4096, ws=ctypes.c_void_p(0x50000),
                 ws_bytes=need - 1) == E.SG_ERR_WORKSPACE
    assert _gemm(lib, lda=4096, ldw=4096, K=4096, ws=ctypes.c_void_p(0x50004),
                 ws_bytes=need) == E.SG_ERR_MISALIGNED
    # row strides below K (negative ones included) are refused whatever K is,
    # K == 0 too: the MFMA kernels build 32-bit buffer bounds from them
    assert _gemm(lib, M=17, N=8, K=0, lda=-1, ldw=0) == E.SG_ERR_INVALID_ARG
    assert _gemm(lib, M=17, N=8, K=0, lda=0, ldw=-8) == E.SG_ERR_INVALID_ARG
    assert _gemm(lib, M=100, N=8, K=0, lda=-(1 << 40), ldw=0) == E.SG_ERR_INVALID_ARG
    assert _gemm(lib, M=2, N=8, K=0, lda=-1, ldw=0, A=NUL, W=NUL) == E.SG_ERR_INVALID_ARG
    # empty problems are no-ops
    assert _gemm(lib, M=0) == E.SG_OK
    assert _gemm(lib, N=0) == E.SG_OK
    assert _gemm(lib, M=0, A=NUL, W=NUL, C=NUL) == E.SG_OK


def test_qkvg_validation(lib):
    E = _lib
    assert lib.kda_qkvg_proj(A16, B16, C16, -1, 4096, 7168, NUL, 0, None) == E.SG_ERR_INVALID_ARG
    assert lib.kda_qkvg_proj(A16, B16, C16, 1, 4096, 7164, NUL, 0, None) == E.SG_ERR_UNSUPPORTED
    assert lib.kda_qkvg_proj(NUL, B16, C16, 1, 4096, 7168, NUL, 0, None) == E.SG_ERR_INVALID_ARG
    assert lib.kda_qkvg_proj(A16, B16, C16, 0, 4096, 7168, NUL, 0, None) == E.SG_OK


def _fab(lib, x=A16, w_ab=B16, w_b=C16, f_a=NUL, beta=ctypes.c_void_p(0x60000),
         g1=ctypes.c_void_p(0x70000), M=2, K=7168, n_ab=136, rank=128, n_b=1024, ws=NUL,
         ws_bytes=0):
    return lib.kda_fab_fb_proj(x, w_ab, w_b, f_a, beta, g1, M, K, n_ab, rank, n_b, ws, ws_bytes,
                               None)


def test_fab_fb_validation(lib):
    E = _lib
    assert _fab(lib, rank=0) == E.SG_ERR_INVALID_ARG
    assert _fab(lib, n_ab=128) == E.SG_ERR_INVALID_ARG
    assert _fab(lib, rank=124) == E.SG_ERR_UNSUPPORTED
    assert _fab(lib, rank=520, n_ab=600) == E.SG_ERR_UNSUPPORTED
    assert _fab(lib, M=300) == E.SG_ERR_UNSUPPORTED
    assert _fab(lib, x=NUL) == E.SG_ERR_INVALID_ARG
    assert _fab(lib, beta=NUL) == E.SG_ERR_INVALID_ARG
    assert _fab(lib, g1=NUL) == E.SG_ERR_INVALID_ARG
    assert _fab(lib, w_b=ODD) == E.SG_ERR_MISALIGNED
    assert _fab(lib) == E.SG_ERR_WORKSPACE  # F_A/beta always needs its partials
    assert _fab(lib, M=0) == E.SG_OK


def test_overlap_validation(lib):
    E = _lib
    # M = 1: the Q/K/V/G rows need no workspace and the F_A/beta rows run on
    # the same GEMV in 7 K-ranges; M = 2: the paired tiles split K, so both
    # ranges leave partials.
    need_aux = lib.sg_kda_workspace_bytes(1, 1, 7168, 4096, 136)
    assert need_aux == 3840  # 7 x 1 x 136 fp32, rounded up to 256 bytes
    assert lib.sg_kda_workspace_bytes(1, 2, 7168, 4096, 136) == 7680  # 7 x 2 x 136 fp32, rounded
    assert lib.sg_kda_workspace_bytes(0, 1, 7168, 4096, 136) == 0
    assert lib.sg_kda_workspace_bytes(0, 2, 7168, 4096, 136) == 7 * 2 * 4096 * 4

    def ov(**kw):
        args = dict(x=A16, packed=B16, w_b=C16, qkvg=ctypes.c_void_p(0x80000),
                    beta=ctypes.c_void_p(0x60000), g1=ctypes.c_void_p(0x70000), M=1, K=7168,
                    n_qkvg=4096, n_ab=136, rank=128, n_b=1024, wsm=NUL, wsm_b=0,
                    wsa=ctypes.c_void_p(0x90000), wsa_b=need_aux)
        args.update(kw)
        return lib.kda_projection_overlap(
            args["x"], args["packed"], args["w_b"], args["qkvg"], args["beta"], args["g1"],
            args["M"], args["K"], args["n_qkvg"], args["n_ab"], args["rank"], args["n_b"],
            args["wsm"], args["wsm_b"], args["wsa"], args["wsa_b"], None, None, None, None)

    assert ov(M=-1) == E.SG_ERR_INVALID_ARG
    assert ov(packed=NUL) == E.SG_ERR_INVALID_ARG
    assert ov(qkvg=NUL) == E.SG_ERR_INVALID_ARG
    assert ov(wsa=NUL) == E.SG_ERR_WORKSPACE
    assert ov(M=2) == E.SG_ERR_WORKSPACE            # ws_main missing
    assert ov(rank=100) == E.SG_ERR_UNSUPPORTED
    assert ov(M=0) == E.SG_OK


def test_latent_tail_validation(lib):
    E = _lib
    out = ctypes.c_void_p(0x80000)

    def tail(L=A16, g=B16, eps=1e-6, w=C16, S=NUL, o=out, M=8, d=2048, D=7168):
        return lib.latent_moe_tail(L, g, eps, w, S, o, M, d, D, NUL, 0, None)

    assert tail(eps=0.0) == E.SG_ERR_INVALID_ARG
    assert tail(eps=-1.0) == E.SG_ERR_INVALID_ARG
    assert tail(eps=float("nan")) == E.SG_ERR_INVALID_ARG
    assert tail(eps=float("inf")) == E.SG_ERR_INVALID_ARG
    assert tail(M=-1) == E.SG_ERR_INVALID_ARG
    assert tail(M=257) == E.SG_ERR_UNSUPPORTED
    assert tail(d=2044) == E.SG_ERR_UNSUPPORTED
    assert tail(d=0) == E.SG_ERR_INVALID_ARG
    assert tail(L=NUL) == E.SG_ERR_INVALID_ARG
    assert tail(g=ODD) == E.SG_ERR_MISALIGNED
    assert tail(o=NUL) == E.SG_ERR_INVALID_ARG
    assert tail(S=ctypes.c_void_p(0x90001)) == E.SG_ERR_MISALIGNED
    assert tail(M=0) == E.SG_OK
    assert tail(D=0) == E.SG_OK


def test_noalloc_rejects_beyond_its_array_before_any_gpu_call(lib):
    """kda_projection_noalloc checks its array's size before it touches the
    GPU: a projection whose workspaces exceed SG_NOALLOC_SCRATCH_BYTES returns
    SG_ERR_WORKSPACE (fake pointers: nothing is dereferenced); M = 0 is a
    no-op."""
    M, K, nq, nab = 256, 7168, 4096, 2304
    need = lib.sg_kda_workspace_bytes(0, M, K, nq, nab) + lib.sg_kda_workspace_bytes(1, M, K, nq, nab)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    args = (A16, B16, C16, ctypes.c_void_p(0x80000), ctypes.c_void_p(0x60000),
            ctypes.c_void_p(0x70000))
    assert lib.kda_projection_noalloc(*args, M, K, nq, nab, 128, 1024, None, None, None,
                                      None) == _lib.SG_ERR_WORKSPACE
    assert lib.kda_projection_noalloc(*args, 0, K, 4096, nab, 128, 1024, None, None, None,
                                      None) == _lib.SG_OK
    assert lib.kda_projection_noalloc(*args, -1, K, 4096, nab, 128, 1024, None, None, None,
                                      None) == _lib.SG_ERR_INVALID_ARG


def test_fab_fb_fused_validates_like_fab_fb(lib):
    """kda_fab_fb_proj_fused takes kda_fab_fb_proj's arguments and checks
    them the same way, before anything is enqueued."""
    def fused(**kw):
        args = dict(x=A16, w_ab=B16, w_b=C16, f_a=NUL, beta=ctypes.c_void_p(0x60000),
                    g1=ctypes.c_void_p(0x70000), M=2, K=7168, n_ab=136, rank=128, n_b=1024,
                    ws=NUL, ws_bytes=0)
        args.update(kw)
        return lib.kda_fab_fb_proj_fused(*args.values(), None)

    E = _lib
    for kw in ({"rank": 0}, {"n_ab": 128}, {"rank": 124}, {"M": 300}, {"x": NUL}, {"g1": NUL},
               {"w_b": ODD}, {}, {"M": 0}, {"ws": ctypes.c_void_p(0x90000), "ws_bytes": 100}):
        assert fused(**kw) == _fab(lib, **kw), kw
    assert fused() == E.SG_ERR_WORKSPACE


def test_one_launch_fits_and_workspace(lib):
    """kda_projection_fused's geometry query and workspace size, restated from
    the header's conditions: one launch at 1 <= M <= 16 for the KDA shapes
    (K <= 8192, n_ab % 4 == 0, rank <= 128, enough Q/K/V/G workgroups for the
    F_A/beta units and F_B hosts), the one-stream schedule elsewhere; the
    workspace is the header plus the larger of the tagged partials
    (ceil(ceil(K/512)/4) K-ranges x M x n_ab x 8 bytes) and the one-stream
    schedule's two workspaces."""
    fits = lambda *a: bool(lib.sg_kda_one_launch_fits(*a))  # noqa: E731
    for M in range(0, 20):
        assert fits(M, 7168, 4096, 136, 128, 1024) == (1 <= M <= 16), M
    assert fits(8, 8192, 4096, 136, 128, 1024)
    assert not fits(8, 8200, 4096, 136, 128, 1024)     # five K-ranges
    assert not fits(4, 7168, 4096, 138, 128, 1024)     # n_ab % 4
    assert not fits(4, 7168, 4096, 136, 256, 1024)     # rank > 128
    assert not fits(4, 7168, 2048, 136, 128, 1024)     # 128 workgroups < 136 units + 16 hosts
    assert fits(8, 7168, 2432, 136, 128, 1024)          # 152 workgroups = 136 units + 16 hosts
    assert not fits(8, 7168, 2416, 136, 128, 1024)
    assert fits(12, 7168, 2688, 136, 128, 1024)         # 168 workgroups = 136 units + 32 hosts
    assert not fits(12, 7168, 2672, 136, 128, 1024)
    assert fits(12, 7168, 4096, 144, 128, 1024)          # a host polls 8 x 144 / 2 = 576 pieces
    assert not fits(12, 7168, 4096, 148, 128, 1024)
    assert not fits(4, 7164, 4096, 136, 128, 1024)     # K % 8
    assert fits(2, 1032, 4096, 136, 128, 1024) and fits(3, 4096, 4096, 136, 128, 1024)
    for M in (1, 2, 5, 8, 9, 16, 40):
        for K in (1032, 4096, 7168):
            ranges = -(-(-(-K // 512)) // 4)
            one = -(-ranges * M * 136 * 8 // 256) * 256
            two = lib.sg_kda_workspace_bytes(0, M, K, 4096, 136) + lib.sg_kda_workspace_bytes(1, M, K, 4096, 136)
            assert lib.sg_kda_workspace_bytes(_lib.SG_KDA_ONE_LAUNCH, M, K, 4096, 136) == \
                _lib.SG_FAB_HEADER_BYTES + max(one, two), (M, K)


def test_projection_fused_validation(lib):
    """kda_projection_fused checks its arguments before anything is enqueued:
    the same statuses as kda_projection_overlap for bad shapes and operands,
    and a workspace of sg_kda_workspace_bytes(SG_KDA_ONE_LAUNCH, ...) bytes."""
    E = _lib
    need = lib.sg_kda_workspace_bytes(E.SG_KDA_ONE_LAUNCH, 4, 7168, 4096, 136)

    def fp(**kw):
        args = dict(x=A16, packed=B16, w_b=C16, qkvg=ctypes.c_void_p(0x80000),
                    beta=ctypes.c_void_p(0x60000), g1=ctypes.c_void_p(0x70000), M=4, K=7168,
                    n_qkvg=4096, n_ab=136, rank=128, n_b=1024, ws=ctypes.c_void_p(0x90000),
                    ws_bytes=need)
        args.update(kw)
        return lib.kda_projection_fused(*args.values(), None)

    assert fp(M=-1) == E.SG_ERR_INVALID_ARG
    assert fp(rank=0) == E.SG_ERR_INVALID_ARG
    assert fp(rank=100) == E.SG_ERR_UNSUPPORTED
    assert fp(x=NUL) == E.SG_ERR_INVALID_ARG
    assert fp(packed=ODD) == E.SG_ERR_MISALIGNED
    assert fp(g1=NUL) == E.SG_ERR_INVALID_ARG
    assert fp(ws=NUL) == E.SG_ERR_WORKSPACE
    assert fp(ws_bytes=need - 1) == E.SG_ERR_WORKSPACE
    assert fp(ws=ctypes.c_void_p(0x90008)) == E.SG_ERR_MISALIGNED
    assert fp(M=0) == E.SG_OK
    # Shapes the one launch does not fit take the one-stream schedule and its checks.
    assert fp(M=20, ws_bytes=100) == E.SG_ERR_WORKSPACE
    assert fp(M=20, qkvg=NUL) == E.SG_ERR_INVALID_ARG


def test_tail_fused_validation_and_workspace(lib):
    """latent_moe_tail_fused validates like latent_moe_tail (the same status
    for every bad argument, before anything is enqueued) and needs the
    hand-off header plus latent_moe_tail's workspace plus, where the GEMM
    sums its two K splits in the launch (17 <= M <= 64 at these shapes),
    8 KiB per 64-row tile and 16-row activation block."""
    E = _lib
    for M in (1, 2, 16, 17, 40, 64, 65, 128, 256):
        base = lib.sg_workspace_bytes(E.SG_OP_LATENT_TAIL, M, 7168, 2048)
        pairs = 112 * -(-M // 16) * 8192 if 17 <= M <= 64 else 0
        assert lib.sg_workspace_bytes(E.SG_OP_LATENT_TAIL_FUSED, M, 7168, 2048) == \
            E.SG_FAB_HEADER_BYTES + base + pairs, M

    def tails(fn, **kw):
        args = dict(L=A16, g=B16, eps=1e-6, w=C16, S=NUL, out=ctypes.c_void_p(0x70000), M=20,
                    d=2048, D=7168, ws=NUL, wsb=0)
        args.update(kw)
        return fn(args["L"], args["g"], ctypes.c_float(args["eps"]), args["w"], args["S"], args["out"],
                  args["M"], args["d"], args["D"], args["ws"], args["wsb"], None)

    for kw in ({"M": -1}, {"eps": 0.0}, {"eps": float("nan")}, {"L": NUL}, {"w": ODD}, {"out": NUL},
               {"d": 0}, {"M": 0}, {}, {"ws": ctypes.c_void_p(0x90008), "wsb": 1 << 24}):
        assert tails(lib.latent_moe_tail_fused, **kw) == tails(lib.latent_moe_tail, **kw), kw
    need = lib.sg_workspace_bytes(E.SG_OP_LATENT_TAIL_FUSED, 20, 7168, 2048)
    assert tails(lib.latent_moe_tail_fused, ws=ctypes.c_void_p(0x90000), wsb=need - 1) == E.SG_ERR_WORKSPACE
