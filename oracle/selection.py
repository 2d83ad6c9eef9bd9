"""Configuration-selection and overlap-gate oracle.

TEST INFRASTRUCTURE ONLY.  An independent transcription, in plain Python, of the
selection rule this library specifies for itself (the table is this library's
own: the reference's ShapeDynamicSkinnyGemm._config in "Kimi K3 support, phase
1", skinny_gemm.py, and KDA_PROJECTION_OVERLAP_MAX_TOKENS / the forward gate in
"Overlap low-M TP8 KDA projections", were tuned for other hardware).  The C++
dispatcher must agree with it field by field.

Rule, for C[M,N] = A[M,K] W[N,K]^T:
  * M, N or K negative -> INVALID_ARG.  K not a multiple of 8 -> UNSUPPORTED.
    M > 256 -> UNSUPPORTED.  M == 0 or N == 0 -> kind NONE, every field 0.
  * Otherwise waves = 4 and nt_weights = 1, and
  * M <= 16, K <= 256: GEMV_SMALLK.  G = smallest power of two >= max(K/8, 1)
    lanes per weight row; rows = 64 / G rows per wave; k_split = 1;
    k_unroll = 1; grid = ceil(N / (4 * rows)); m_tile = M.
  * M <= 16, K > 256: steps = ceil((K/8) / 64).
      - N >= 1024: GEMV_ROW, rows = 1 (M <= 2), 2 (M <= 8) or 4; want = 1.
      - N < 1024: GEMV_SPLITK, rows = 1, want = ceil(2048 / N).
      depth = 16, 14, 7 for rows = 1, 2, 4 (k_unroll = depth);
      max_sps = min(floor(128 / M), depth), need = ceil(steps / max_sps),
      k_split = split(steps, max(want, need)), sps = ceil(steps / k_split);
      waves = 8 if M * sps > 64 else 4.
      grid = ceil(N / (waves * rows)) * k_split; m_tile = M.
  * 17 <= M <= 256: MFMA_TILE, m_tile = 16 * ceil(M / 16), rows = 1,
    k_unroll = 12, 8, 4, 2 for m_tile/16 <= 2, <= 4, <= 8, above;
    tiles = ceil(N / 16), ksteps = ceil(K / 32).
      - tiles >= 192: k_split = 1.
      - else want = min(ceil(256 / tiles), max(1, floor(ksteps / 8))),
        k_split = split(ksteps, want).
    grid = tiles * k_split.
  * split(steps, want): 1 if steps <= 0 or want <= 1; else with
    w = min(want, steps) and per = ceil(steps / w), ceil(steps / per).

Overlap gate: enabled and 0 < M <= 32 and x contiguous and an aux stream and
the event pair are present.
"""
from __future__ import annotations

OK, INVALID_ARG, UNSUPPORTED = 0, -1, -2
NONE, GEMV_ROW, GEMV_SPLITK, GEMV_SMALLK, MFMA_TILE = 0, 1, 2, 3, 4
OVERLAP_MAX_TOKENS = 32

FIELDS = ("kind", "m_tile", "rows", "waves", "k_split", "k_unroll", "grid", "nt_weights")


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _split(steps: int, want: int) -> int:
    if steps <= 0 or want <= 1:
        return 1
    w = min(want, steps)
    per = _cdiv(steps, w)
    return _cdiv(steps, per)


def select(M: int, N: int, K: int, has_residual: bool = False):
    """Returns (status, config dict or None)."""
    if M < 0 or N < 0 or K < 0:
        return INVALID_ARG, None
    if K % 8:
        return UNSUPPORTED, None
    if M > 256:
        return UNSUPPORTED, None
    cfg = dict.fromkeys(FIELDS, 0)
    if M == 0 or N == 0:
        return OK, cfg
    cfg["waves"] = 4
    cfg["nt_weights"] = 1
    if M <= 16:
        cfg["m_tile"] = M
        if K <= 256:
            g = 1
            while g < max(K // 8, 1):
                g *= 2
            cfg.update(kind=GEMV_SMALLK, rows=64 // g, k_split=1, k_unroll=1)
            cfg["grid"] = _cdiv(N, 4 * cfg["rows"])
        else:
            steps = _cdiv(K // 8, 64)
            if N >= 1024:
                rows = 1 if M <= 2 else (2 if M <= 8 else 4)
                cfg.update(kind=GEMV_ROW, rows=rows)
                want = 1
            else:
                cfg.update(kind=GEMV_SPLITK, rows=1)
                want = _cdiv(2048, N)
            depth = {1: 16, 2: 14, 4: 7}[cfg["rows"]]
            max_sps = min(128 // M, depth)
            need = _cdiv(steps, max_sps)
            cfg["k_split"] = _split(steps, max(want, need))
            sps = _cdiv(steps, cfg["k_split"])
            cfg["waves"] = 8 if M * sps > 64 else 4
            cfg["k_unroll"] = depth
            cfg["grid"] = _cdiv(N, cfg["waves"] * cfg["rows"]) * cfg["k_split"]
    else:
        tiles = _cdiv(N, 16)
        ksteps = _cdiv(K, 32)
        if tiles >= 192:
            ks = 1
        else:
            want = min(_cdiv(256, tiles), max(1, ksteps // 8))
            ks = _split(ksteps, want)
        mb = _cdiv(M, 16)
        depth = 12 if mb <= 2 else (8 if mb <= 4 else (4 if mb <= 8 else 2))
        cfg.update(kind=MFMA_TILE, m_tile=16 * mb, rows=1, k_unroll=depth, k_split=ks,
                   grid=tiles * ks)
    return OK, cfg


def overlap_gate(M: int, x_contiguous: bool, have_aux: bool, have_events: bool,
                 enabled: bool = True) -> bool:
    return bool(enabled and 0 < M <= OVERLAP_MAX_TOKENS and x_contiguous and have_aux
                and have_events)
