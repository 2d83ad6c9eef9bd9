"""Configuration-selection and overlap-gate oracle.

TEST INFRASTRUCTURE ONLY.  An independent transcription, in plain Python, of the
selection rule this library specifies for itself (the table is this library's
own: the reference's ShapeDynamicSkinnyGemm._config in "Kimi K3 support, phase
1", skinny_gemm.py, and KDA_PROJECTION_OVERLAP_MAX_TOKENS / the forward gate in
"Overlap low-M TP8 KDA projections", were tuned for other hardware).  The C++
dispatcher must agree with it field by field.

The measured table: bf16_skinny_gemm_02_amd/tuned_table.json (written by the
tuner from its own measurements; data, not code).  Where one of its chosen
entries has this N and K and m_lo <= M <= m_hi, the entry's kind, rows,
waves, k_unroll and k_split replace the rule's, with m_tile 4 ceil(M / 4)
(MFMA_WAVESPLIT; MFMA_TILE with 2 waves), 16 ceil(M / 16) (MFMA_TILE with 4
waves), 128 ceil(M / 128) (MFMA_BLOCK) or M (the GEMV kinds), and grid
ceil(N / (waves rows)) k_split (GEMV), ceil(N / 64) ceil(M / 128) k_split
(BLOCK) or ceil(N / rows) k_split; the gate's OVERLAP_MAX_TOKENS is the
table's overlap.max_tokens (0 without a table).

Rule, for C[M,N] = A[M,K] W[N,K]^T:
  * M, N or K negative -> INVALID_ARG.  K not a multiple of 8 -> UNSUPPORTED.
    M > 256 -> UNSUPPORTED.  M == 0 or N == 0 -> kind NONE, every field 0.
  * Otherwise nt_weights = 1, waves = 4 unless stated, ksteps = ceil(K / 32),
    and
  * M <= 16, K <= 256: GEMV_SMALLK.  G = smallest power of two >= max(K/8, 1)
    lanes per weight row; rows = 64 / G rows per wave; k_split = 1;
    k_unroll = 1; grid = ceil(N / (4 * rows)); m_tile = M.
  * M == 1 (K > 256): steps = ceil((K/8) / 64).
      - N >= 1024: GEMV_ROW, want = 1.
      - N < 1024: GEMV_SPLITK, want = ceil(2048 / N).
      need = ceil(steps / 16), k_split = split(steps, max(want, need)),
      m_tile = 1, rows = 7 if GEMV_ROW and steps <= 4, else 4 if GEMV_ROW and
      steps <= 7, else 1, k_unroll = 16,
      grid = ceil(N / (4 * rows)) * k_split.
  * 2 <= M <= 16: m_tile = 4 * ceil(M / 4), tiles16 = ceil(N / 16),
    wide = 4 * ceil(ceil(N / 256) / 4).
      - tiles16 > 320 and wide <= 32: MFMA_WAVESPLIT, rows = wide, waves = 4,
        k_unroll = 3, k_split = msplit(ceil(N / wide), 16), grid =
        ceil(N / wide) * k_split.
      - tiles16 <= 320, or m_tile <= 8 and tiles16 <= 512: MFMA_WAVESPLIT,
        rows = 16, waves = 4, k_unroll = 3, k_split = msplit(tiles16, 16),
        grid = tiles16 * k_split.
      - else tiles16 <= 512: the same with k_unroll = 2.
      - else MFMA_TILE, rows = 32, waves = 2, k_unroll = 4,
        tiles = ceil(N / 32), k_split = msplit(tiles, 8), grid = tiles * k_split.
  * 17 <= M <= 64: MFMA_TILE, m_tile = 16 * ceil(M / 16), rows = 64, waves = 4,
    k_unroll = 3, tiles = ceil(N / 64), k_split = msplit(tiles, 8),
    grid = tiles * k_split.
  * 65 <= M <= 256: MFMA_BLOCK, m_tile = 128 * ceil(M / 128), rows = 64,
    waves = 4, k_unroll = 3, tiles = ceil(N / 64) * ceil(M / 128),
    k_split = msplit(tiles, 8), grid = tiles * k_split.
  * msplit(tiles, min_steps): 1 if tiles >= 192; else
    split(ksteps, min(ceil(224 / tiles), max(1, floor(ksteps / min_steps)))).
  * split(steps, want): 1 if steps <= 0 or want <= 1; else with
    w = min(want, steps) and per = ceil(steps / w), ceil(steps / per).

Overlap gate: enabled and 0 < M <= OVERLAP_MAX_TOKENS and x contiguous and an
aux stream and the event pair are present.

KDA projection row ranges (kda_select; which = 0 Q/K/V/G and 1 F_A/beta in the
packed projection, 2 F_A/beta alone):
  * f = select(M, n_ab, K); a GEMV_SMALLK f becomes, with k_split = 1,
    GEMV_SPLITK (M == 1: m_tile 1, rows 1, waves 4, k_unroll 16,
    grid ceil(n_ab / 4)) or MFMA_WAVESPLIT (M > 1: m_tile 4 ceil(M / 4),
    rows 16, waves 4, k_unroll 3, grid ceil(n_ab / 16)); k_split >= 1;
    more than 8 K-ranges are cut to split(steps, max(need, 8)), steps =
    ceil((K/8) / 64) and need = ceil(steps / 16) for the GEMV kinds, steps =
    ceil(K / 32) and need = 1 otherwise, grid scaled to match.
  * which 2: f.  Otherwise q = select(M, n_qkvg, K).  If q is GEMV_ROW with
    k_split 1, f becomes q's configuration with kind GEMV_SPLITK, k_split =
    split(ceil((K/8) / 64), 7) and grid ceil(n_ab / (4 rows)) * k_split.
    Else, if q and f are both
    MFMA_WAVESPLIT or MFMA_TILE: with t_q = ceil(n_qkvg / 128), t_f =
    ceil(n_ab / 128), ksteps = ceil(K / 32), S = split(ksteps,
    min(256 // (t_q + t_f), max(1, ksteps // 8))), both become MFMA_TILE with
    m_tile 4 ceil(M / 4) (M <= 16) or 16 ceil(M / 16), rows 128, waves 8,
    k_unroll 3, k_split S, grid t * S.
  * workspace: Q/K/V/G k_split * M * n_qkvg * 4 (0 when k_split <= 1),
    F_A/beta k_split * M * n_ab * 4, each rounded up to 256.
"""
from __future__ import annotations

OK, INVALID_ARG, UNSUPPORTED = 0, -1, -2
NONE, GEMV_ROW, GEMV_SPLITK, GEMV_SMALLK, MFMA_TILE, MFMA_WAVESPLIT, MFMA_BLOCK = 0, 1, 2, 3, 4, 5, 6

def _load_table():
    import json
    from pathlib import Path
    path = Path(__file__).resolve().parent.parent / "bf16_skinny_gemm_02_amd" / "tuned_table.json"
    if not path.exists():
        return [], 0
    t = json.loads(path.read_text())
    entries = []
    for b in t["buckets"]:
        e = {"N": b["N"], "K": b["K"], "m_lo": b["m_lo"], "m_hi": b["m_hi"]}
        e.update({f: int(b["chosen"][f]) for f in ("kind", "rows", "waves", "k_unroll", "k_split")})
        entries.append(e)
    return entries, int(t["overlap"]["max_tokens"])


TABLE, OVERLAP_MAX_TOKENS = _load_table()

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
    ksteps = _cdiv(K, 32)

    def msplit(tiles: int, min_steps: int) -> int:
        if tiles >= 192:
            return 1
        cap = max(1, ksteps // min_steps)
        return _split(ksteps, min(_cdiv(224, tiles), cap))

    if M <= 16 and K <= 256:
        g = 1
        while g < max(K // 8, 1):
            g *= 2
        cfg.update(kind=GEMV_SMALLK, m_tile=M, rows=64 // g, k_split=1, k_unroll=1)
        cfg["grid"] = _cdiv(N, 4 * cfg["rows"])
    elif M == 1:
        steps = _cdiv(K // 8, 64)
        if N >= 1024:
            kind, want = GEMV_ROW, 1
        else:
            kind, want = GEMV_SPLITK, _cdiv(2048, N)
        ks = _split(steps, max(want, _cdiv(steps, 16)))
        rows = 7 if (kind == GEMV_ROW and steps <= 4) else (4 if (kind == GEMV_ROW and steps <= 7) else 1)
        cfg.update(kind=kind, m_tile=1, rows=rows, k_split=ks, k_unroll=16,
                   grid=_cdiv(N, 4 * rows) * ks)
    elif M <= 16:
        cfg["m_tile"] = 4 * _cdiv(M, 4)
        tiles16 = _cdiv(N, 16)
        wide = 4 * _cdiv(_cdiv(N, 256), 4)
        if tiles16 > 320 and wide <= 32:
            tiles = _cdiv(N, wide)
            ks = msplit(tiles, 16)
            cfg.update(kind=MFMA_WAVESPLIT, rows=wide, waves=4, k_unroll=3, k_split=ks,
                       grid=tiles * ks)
        elif tiles16 <= 320 or (cfg["m_tile"] <= 8 and tiles16 <= 512):
            ks = msplit(tiles16, 16)
            cfg.update(kind=MFMA_WAVESPLIT, rows=16, waves=4, k_unroll=3, k_split=ks,
                       grid=tiles16 * ks)
        elif tiles16 <= 512:
            ks = msplit(tiles16, 16)
            cfg.update(kind=MFMA_WAVESPLIT, rows=16, waves=4, k_unroll=2, k_split=ks,
                       grid=tiles16 * ks)
        else:
            tiles = _cdiv(N, 32)
            ks = msplit(tiles, 8)
            cfg.update(kind=MFMA_TILE, rows=32, waves=2, k_unroll=4, k_split=ks,
                       grid=tiles * ks)
    elif M <= 64:
        tiles = _cdiv(N, 64)
        ks = msplit(tiles, 8)
        cfg.update(kind=MFMA_TILE, m_tile=16 * _cdiv(M, 16), rows=64, waves=4, k_unroll=3,
                   k_split=ks, grid=tiles * ks)
    else:
        tiles = _cdiv(N, 64) * _cdiv(M, 128)
        ks = msplit(tiles, 8)
        cfg.update(kind=MFMA_BLOCK, m_tile=128 * _cdiv(M, 128), rows=64, k_unroll=3, k_split=ks,
                   grid=tiles * ks)
    for e in TABLE:
        if e["N"] == N and e["K"] == K and e["m_lo"] <= M <= e["m_hi"]:
            return OK, _from_entry(e, M, N)
    return OK, cfg


def _from_entry(e: dict, M: int, N: int) -> dict:
    kind, rows, waves, S = e["kind"], e["rows"], e["waves"], e["k_split"]
    if kind == MFMA_WAVESPLIT or (kind == MFMA_TILE and waves == 2):
        m_tile = 4 * _cdiv(M, 4)
    elif kind == MFMA_TILE:
        m_tile = 16 * _cdiv(M, 16)
    elif kind == MFMA_BLOCK:
        m_tile = 128 * _cdiv(M, 128)
    else:
        m_tile = M
    if kind in (GEMV_ROW, GEMV_SPLITK):
        grid = _cdiv(N, waves * rows) * S
    elif kind == GEMV_SMALLK:
        grid = _cdiv(N, waves * rows)
    elif kind == MFMA_BLOCK:
        grid = _cdiv(N, 64) * _cdiv(M, 128) * S
    else:
        grid = _cdiv(N, rows) * S
    return dict(kind=kind, m_tile=m_tile, rows=rows, waves=waves, k_split=S, k_unroll=e["k_unroll"],
                grid=grid, nt_weights=1)


def overlap_gate(M: int, x_contiguous: bool, have_aux: bool, have_events: bool,
                 enabled: bool = True) -> bool:
    return bool(enabled and 0 < M <= OVERLAP_MAX_TOKENS and x_contiguous and have_aux
                and have_events)


def kda_select(which: int, M: int, K: int, n_qkvg: int, n_ab: int):
    """Returns (status, config dict or None) for one row range of the KDA projection."""
    if which not in (0, 1, 2) or M < 0 or K < 0 or n_qkvg < 0 or n_ab < 0:
        return INVALID_ARG, None
    st, q = select(M, n_qkvg, K)
    if st != OK:
        return st, None
    st, f = select(M, n_ab, K)
    if st != OK:
        return st, None
    if f["kind"] == GEMV_SMALLK:
        if M == 1:
            f.update(kind=GEMV_SPLITK, m_tile=1, rows=1, waves=4, k_unroll=16, grid=_cdiv(n_ab, 4))
        else:
            f.update(kind=MFMA_WAVESPLIT, m_tile=4 * _cdiv(M, 4), rows=16, waves=4, k_unroll=3,
                     grid=_cdiv(n_ab, 16))
        f["k_split"] = 1
    f["k_split"] = max(f["k_split"], 1)
    if f["k_split"] > 8:
        gemv = f["kind"] in (GEMV_SPLITK, GEMV_ROW)
        steps = _cdiv(K // 8, 64) if gemv else _cdiv(K, 32)
        need = _cdiv(steps, 16) if gemv else 1
        tiles = f["grid"] // f["k_split"]
        f["k_split"] = _split(steps, max(need, 8))
        f["grid"] = tiles * f["k_split"]
    if which == 2:
        return OK, f
    if q["kind"] == GEMV_ROW and q["k_split"] == 1:
        ks = _split(_cdiv(K // 8, 64), 7)
        f = dict(q, kind=GEMV_SPLITK, k_split=ks, grid=_cdiv(n_ab, q["waves"] * q["rows"]) * ks)
    small = (MFMA_WAVESPLIT, MFMA_TILE)
    if q["kind"] in small and f["kind"] in small:
        tq, tf = _cdiv(n_qkvg, 128), _cdiv(n_ab, 128)
        ksteps = _cdiv(K, 32)
        S = _split(ksteps, min(256 // (tq + tf), max(1, ksteps // 8)))
        mt = 4 * _cdiv(M, 4) if M <= 16 else 16 * _cdiv(M, 16)
        for c, t in ((q, tq), (f, tf)):
            c.update(kind=MFMA_TILE, m_tile=mt, rows=128, waves=8, k_unroll=3, k_split=S,
                     grid=t * S)
    return OK, (q if which == 0 else f)


def kda_workspace_bytes(which: int, M: int, K: int, n_qkvg: int, n_ab: int) -> int:
    if M <= 0 or K < 0 or n_qkvg < 0 or n_ab <= 0 or which not in (0, 1):
        return 0
    st, c = kda_select(which, M, K, n_qkvg, n_ab)
    if st != OK or c["kind"] == NONE:
        return 0
    if which == 0 and c["k_split"] <= 1:
        return 0
    n = n_qkvg if which == 0 else n_ab
    return -(-(c["k_split"] * M * n * 4) // 256) * 256
