"""Measure the configuration table and the overlap gate on this GPU, and emit them.

    python -m bf16_skinny_gemm_02_amd.tune [--shapes qkvg,fab,fb,tail,packed] [--reps 10]
    python -m bf16_skinny_gemm_02_amd.tune --emit     # re-render from the measured table

The analogue of the load-time autotune of the KDA projection ("Overlap low-M
TP8 KDA projections", autotune_kda_qkvg: measure the candidate configurations
per shape, keep the fastest, derive the overlap limit from measurement) and of
the test that the configs in use equal the measured table
(test_kda_overlap_configs_match_measured_table).

For each of the five (N, K) shapes on the path -- Q/K/V/G [4096, 7168],
F_A/beta [136, 7168], F_B [1024, 128], the latent-MoE up-projection
[7168, 2048] and the packed projection weight [4232, 7168] -- and each range
of M that shares kernel instances (BUCKETS), every candidate configuration
the kernels support (sg_config_supported) is installed as the library's
override table (sg_set_table_override) and timed through the entry point
that serves the shape, at both ends of the range: a hipGraph of back-to-back
calls over weight copies spanning >= 512 MiB (cold weights; at most 64
copies), replayed and timed with HIP events.  The candidate with the least
total time wins, unless the incumbent (the library's choice before the run)
is within MARGIN of it.  The overlap gate is then measured as
tune_gate does, with the winners installed.

Outputs (--out-dir, default: this package):
  tuned_table.json        the measured table: every candidate's times, the
                          incumbent, the winner, the gate measurement
  csrc/tuned_table.inc    the compiled table (rebuild the library after)
  ../docs/config_table.md the table for readers
"""
from __future__ import annotations

import argparse
import json
import math
import time
from pathlib import Path

PKG = Path(__file__).resolve().parent
JSON_PATH = PKG / "tuned_table.json"
INC_PATH = PKG / "csrc" / "tuned_table.inc"
MD_PATH = PKG.parent / "docs" / "config_table.md"

GEMV_ROW, GEMV_SPLITK, GEMV_SMALLK, MFMA_TILE, MFMA_WAVESPLIT, MFMA_BLOCK = 1, 2, 3, 4, 5, 6
KIND_NAMES = {1: "GEMV_ROW", 2: "GEMV_SPLITK", 3: "GEMV_SMALLK", 4: "MFMA_TILE",
              5: "MFMA_WAVESPLIT", 6: "MFMA_BLOCK"}
FIELDS = ("kind", "rows", "waves", "k_unroll", "k_split")
ENTRY_FIELDS = ("N", "K", "m_lo", "m_hi") + FIELDS

# name: (N, K, entry point that serves the shape)
SHAPES = {
    "qkvg": (4096, 7168, "kda_qkvg_proj"),
    "fab": (136, 7168, "kda_fab_fb_proj"),
    "fb": (1024, 128, "skinny_gemm"),
    "tail": (7168, 2048, "latent_moe_tail"),
    "packed": (4232, 7168, "skinny_gemm"),
}
# Ranges of M that share kernel instances (activation tiles of 4, 16, 128 rows).
BUCKETS = ((1, 1), (2, 4), (5, 8), (9, 12), (13, 16), (17, 32), (33, 48), (49, 64),
           (65, 128), (129, 256))
MARGIN = 0.02           # the incumbent stays unless a candidate is > 2% faster in total
COLD_BYTES = 512 << 20  # weight copies per graph span at least this (Infinity Cache: 256 MiB)
MAX_COPIES = 64
GATE_MS = (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64)


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _eff(steps: int, want: int) -> int:
    """Non-empty ranges when `steps` units are cut into at most `want` equal ranges."""
    if steps <= 0 or want <= 1:
        return 1
    want = min(want, steps)
    return _cdiv(steps, _cdiv(steps, want))


def candidates(N: int, K: int, lo: int, hi: int) -> list:
    """Configurations (kind, rows, waves, k_unroll, k_split) worth timing for
    N x K at lo <= M <= hi; the library's sg_config_supported filters them."""
    ks = _cdiv(K, 32)              # 32-wide MFMA k-steps
    steps = _cdiv(K // 8, 64)      # 512-wide GEMV steps
    out = []

    def add(kind, rows, waves, k_unroll, k_split):
        c = dict(kind=kind, rows=rows, waves=waves, k_unroll=k_unroll, k_split=k_split)
        if c not in out:
            out.append(c)

    if hi == 1:
        kind = GEMV_ROW if N >= 1024 else GEMV_SPLITK
        for rows in (1, 4, 7):
            for s in (1, 2, 4, 7, 8, 14):
                add(kind, rows, 4, 16, _eff(steps, s))
    if hi <= 16:
        wide = 4 * _cdiv(_cdiv(N, 256), 4)
        shapes = [(16, 3), (16, 2), (32, 3)]
        if 16 < wide < 32:
            shapes.append((wide, 3))
        for s in (1, 2, 4, 8):
            for rows, ring in shapes:
                add(MFMA_WAVESPLIT, rows, 4, ring, _eff(ks, s))
            add(MFMA_TILE, 32, 2, 4, _eff(ks, s))
    if lo >= 17 and hi <= 64:
        for s in (1, 2, 3, 4, 7, 8, 14):
            add(MFMA_TILE, 64, 4, 3, _eff(ks, s))
        for s in (1, 2, 4, 7, 8, 14):  # 8 waves, 128 rows: the packed projection's tile
            add(MFMA_TILE, 128, 8, 3, _eff(ks, s))
    if lo >= 17:
        for s in (1, 2, 4, 7, 8):
            add(MFMA_BLOCK, 64, 4, 3, _eff(ks, s))
    return out


def key(c: dict) -> tuple:
    return tuple(int(c[f]) for f in FIELDS)


def choose(cands: list, incumbent: dict, margin: float = MARGIN) -> dict:
    """The winner among measured candidates ({"cfg", "total_us"}; total_us None
    when the candidate failed): the fastest, unless the incumbent's total is
    within `margin` of it."""
    ok = [c for c in cands if c.get("total_us") is not None]
    if not ok:
        return dict(incumbent)
    best = min(ok, key=lambda c: (c["total_us"], key(c["cfg"])))
    inc = [c for c in ok if key(c["cfg"]) == key(incumbent)]
    if inc and inc[0]["total_us"] <= best["total_us"] * (1.0 + margin):
        return dict(inc[0]["cfg"])
    return dict(best["cfg"])


def table_entries(table: dict) -> list:
    """The compiled entries, in file order: one per (shape, bucket)."""
    out = []
    for b in table["buckets"]:
        e = {"N": b["N"], "K": b["K"], "m_lo": b["m_lo"], "m_hi": b["m_hi"]}
        e.update({f: int(b["chosen"][f]) for f in FIELDS})
        out.append(e)
    return out


def render_inc(table: dict) -> str:
    lines = [
        "// The measured configuration table, written by `python -m",
        "// bf16_skinny_gemm_02_amd.tune` from its measured table",
        "// (bf16_skinny_gemm_02_amd/tuned_table.json); do not edit by hand.",
        "// Columns: N, K, m_lo, m_hi, kind, rows, waves, k_unroll, k_split.",
    ]
    entries = table_entries(table)
    if not entries:
        lines.append("// No entries: one sentinel (N = 0 matches no problem).")
        entries = [{f: 0 for f in ENTRY_FIELDS}]
    lines.append("const sg_table_entry_t kTunedTable[] = {")
    for e in entries:
        lines.append("    {" + ", ".join(str(int(e[f])) for f in ENTRY_FIELDS) + "},")
    lines.append("};")
    lines.append(f"constexpr int kTunedOverlapMaxTokens = {int(table['overlap']['max_tokens'])};")
    return "\n".join(lines) + "\n"


def _cfg_text(c: dict) -> str:
    return f"{KIND_NAMES.get(int(c['kind']), c['kind'])} r{c['rows']} w{c['waves']} u{c['k_unroll']} s{c['k_split']}"


def render_md(table: dict) -> str:
    out = ["# Measured configuration table", "",
           "Written by `python -m bf16_skinny_gemm_02_amd.tune` from `bf16_skinny_gemm_02_amd/tuned_table.json`;",
           "compiled into the library as `csrc/tuned_table.inc`. µs per call at the two ends of each range",
           f"of M (graph replay, cold weights). Device: {table.get('device', '?')}. "
           f"Policy: the incumbent stays unless a candidate is more than {100 * table.get('margin', MARGIN):.0f}% faster in total.",
           "", "| shape | N x K | M | incumbent | µs | chosen | µs | candidates |",
           "|---|---|---|---|---|---|---|---|"]
    for b in table["buckets"]:
        times = {key(c["cfg"]): c for c in b["candidates"]}
        inc = times.get(key(b["incumbent"]), {})
        ch = times.get(key(b["chosen"]), {})

        def fmt(c):
            us = c.get("us")
            return " / ".join(f"{u:.2f}" for u in us) if us else "—"
        m = f"{b['m_lo']}" if b["m_lo"] == b["m_hi"] else f"{b['m_lo']}..{b['m_hi']}"
        out.append(f"| {b['shape']} | {b['N']} x {b['K']} | {m} | {_cfg_text(b['incumbent'])} | {fmt(inc)} | "
                   f"{_cfg_text(b['chosen'])} | {fmt(ch)} | {len(b['candidates'])} |")
    ov = table["overlap"]
    out += ["", f"Overlap gate: `sg_overlap_max_tokens` = {ov['max_tokens']} (the largest M up to which the "
            "two-stream projection measured faster at every M).", "",
            "| M | one stream µs | two streams µs |", "|---|---|---|"]
    for r in ov.get("per_m", []):
        out.append(f"| {r['M']} | {r['one_stream_us']} | {r['two_stream_us']} |")
    return "\n".join(out) + "\n"


def emit(table: dict, out_dir: Path | None = None) -> None:
    pkg = out_dir or PKG
    pkg.mkdir(parents=True, exist_ok=True)
    (pkg / "tuned_table.json").write_text(json.dumps(table, indent=1) + "\n")
    (pkg / "csrc").mkdir(parents=True, exist_ok=True)
    (pkg / "csrc" / "tuned_table.inc").write_text(render_inc(table))
    md = (pkg.parent / "docs" / "config_table.md") if out_dir else MD_PATH
    md.parent.mkdir(parents=True, exist_ok=True)
    md.write_text(render_md(table))


# ---- measurement (GPU) ---------------------------------------------------------

class _Shape:
    """Inputs, weight copies and the call of one shape."""

    def __init__(self, name, device, gen):
        import torch
        from . import SG_OP_FAB_FB, SG_OP_GEMM, SG_OP_LATENT_TAIL
        self.name = name
        self.N, self.K, self.entry = SHAPES[name]
        self.device = device
        wbytes = 2 * self.N * self.K + (2 * 1024 * 128 if name == "fab" else 0)
        self.R = max(2, min(MAX_COPIES, math.ceil(COLD_BYTES / wbytes)))
        w0 = (torch.randn(self.N, self.K, generator=gen) / math.sqrt(self.K)).to(torch.bfloat16)
        self.w = [w0.to(device) for _ in range(self.R)]
        if name == "fab":
            b0 = (torch.randn(1024, 128, generator=gen) / math.sqrt(128)).to(torch.bfloat16)
            self.w_b = [b0.to(device) for _ in range(self.R)]
        if name == "tail":
            self.gamma = (torch.rand(self.K, generator=gen) + 0.5).to(torch.bfloat16).to(device)
        self.op = {"kda_qkvg_proj": SG_OP_GEMM, "skinny_gemm": SG_OP_GEMM,
                   "kda_fab_fb_proj": SG_OP_FAB_FB, "latent_moe_tail": SG_OP_LATENT_TAIL}[self.entry]
        self.gen = gen

    def make_call(self, M):
        """The call at batch M with its buffers (workspace sized for the
        configuration installed now)."""
        import torch
        from . import (kda_fab_fb_proj, kda_qkvg_proj, latent_moe_tail, sg_workspace_bytes,
                       skinny_gemm)
        dev, N, K = self.device, self.N, self.K
        x = torch.randn(M, K, generator=self.gen).to(torch.bfloat16).to(dev)
        ws = torch.zeros(max(256, sg_workspace_bytes(self.op, M, N, K)), dtype=torch.uint8, device=dev)
        if self.entry == "kda_qkvg_proj":
            out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            return lambda r: kda_qkvg_proj(x, self.w[r], out=out, workspace=ws)
        if self.entry == "skinny_gemm":
            out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            return lambda r: skinny_gemm(x, self.w[r], out=out, workspace=ws)
        if self.entry == "kda_fab_fb_proj":
            g1 = torch.empty(M, 1024, dtype=torch.bfloat16, device=dev)
            beta = torch.empty(M, N - 128, dtype=torch.bfloat16, device=dev)
            return lambda r: kda_fab_fb_proj(x, self.w[r], self.w_b[r], g1=g1, beta=beta, workspace=ws)
        S = torch.randn(M, N, generator=self.gen).to(torch.bfloat16).to(dev)
        out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        return lambda r: latent_moe_tail(x, self.gamma, self.w[r], S, eps=1e-6, out=out, workspace=ws)


def _time_call(fn, R, stream, reps):
    from .tune_gate import _graph, _time
    g = _graph(fn, R, stream)
    ts = sorted(_time(g, stream, reps) * 1000.0 / R for _ in range(3))
    del g
    return ts[1]


def _effective(shape, entry, M):
    """What the serving entry point actually runs at M with `entry` installed
    (the F_A/beta branch derives its own configuration from the table's)."""
    from . import SG_KDA_FAB_ALONE, sg_kda_select, sg_select
    if shape.entry == "kda_fab_fb_proj":
        return tuple(sorted(sg_kda_select(SG_KDA_FAB_ALONE, M, shape.K, 0, shape.N).items()))
    return tuple(sorted(sg_select(M, shape.N, shape.K).items()))


def measure_bucket(shape, lo, hi, stream, reps, log):
    from . import sg_config_supported, sg_select, sg_set_table_override
    from ._lib import SkinnyGemmError
    sg_set_table_override([])
    inc_cfg = sg_select(hi, shape.N, shape.K)
    incumbent = {f: int(inc_cfg[f]) for f in FIELDS}
    cands = candidates(shape.N, shape.K, lo, hi)
    if incumbent not in cands:
        cands.insert(0, incumbent)
    points = (lo,) if lo == hi else (lo, hi)
    results, seen = [], {}
    for c in cands:
        entry = dict(N=shape.N, K=shape.K, m_lo=lo, m_hi=hi, **c)
        ok = all(sg_config_supported(_full(c, M, shape.N), M, shape.N, shape.K) for M in range(lo, hi + 1))
        if not ok:
            continue
        try:
            sg_set_table_override([entry])
        except ValueError:  # not supported at some M of the range
            continue
        eff = tuple(_effective(shape, entry, M) for M in points)
        if eff in seen:  # the serving entry point runs an already measured configuration
            sg_set_table_override([])
            same = seen[eff]
            results.append({"cfg": c, "same_as": same["cfg"], "us": same["us"],
                            "total_us": same["total_us"]})
            continue
        us = []
        try:
            for M in points:
                us.append(round(_time_call(shape.make_call(M), shape.R, stream, reps), 3))
            total = round(sum(us), 3)
        except (ValueError, SkinnyGemmError) as e:
            us, total = None, None
            log(f"[tune] {shape.name} M={lo}..{hi} {c}: {e}")
        finally:
            sg_set_table_override([])
        results.append({"cfg": c, "us": us, "total_us": total})
        seen[eff] = results[-1]
    chosen = choose(results, incumbent)
    return {"shape": shape.name, "N": shape.N, "K": shape.K, "m_lo": lo, "m_hi": hi,
            "measured_at": list(points), "incumbent": incumbent, "chosen": chosen,
            "candidates": results}


def _full(c, M, N):
    """sg_config_t fields of table configuration c at M (m_tile and grid as
    the library derives them)."""
    kind, rows, waves, S = int(c["kind"]), int(c["rows"]), int(c["waves"]), int(c["k_split"])
    if kind == MFMA_WAVESPLIT:
        m_tile = 4 * _cdiv(M, 4)
    elif kind == MFMA_TILE:
        m_tile = 4 * _cdiv(M, 4) if waves == 2 else 16 * _cdiv(M, 16)
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
    return dict(kind=kind, m_tile=m_tile, rows=rows, waves=waves, k_split=S,
                k_unroll=int(c["k_unroll"]), grid=grid, nt_weights=1)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--shapes", default=",".join(SHAPES))
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--emit", action="store_true", help="re-render the .inc and .md from the JSON")
    ap.add_argument("--out-dir", type=Path, default=None)
    args = ap.parse_args()
    if args.emit:
        emit(json.loads(JSON_PATH.read_text()), args.out_dir)
        return
    import torch
    from . import sg_set_table_override
    from .tune_gate import derive_gate, measure
    if not torch.cuda.is_available():
        raise SystemExit("the tuner needs a GPU")
    device = torch.device("cuda:0")
    stream = torch.cuda.Stream(device)
    gen = torch.Generator(device="cpu").manual_seed(20260)
    log = lambda s: print(s, flush=True)  # noqa: E731
    t0 = time.time()
    buckets = []
    for name in [s for s in args.shapes.split(",") if s]:
        shape = _Shape(name, device, gen)
        for lo, hi in BUCKETS:
            b = measure_bucket(shape, lo, hi, stream, args.reps, log)
            buckets.append(b)
            best = [c for c in b["candidates"] if c["cfg"] == b["chosen"]]
            log(f"[tune] {name} M={lo}..{hi}: {len(b['candidates'])} candidates, chosen "
                f"{_cfg_text(b['chosen'])} {best[0]['us'] if best else ''} "
                f"(incumbent {_cfg_text(b['incumbent'])}), {time.time() - t0:.0f} s")
        del shape
        torch.cuda.empty_cache()
    # The gate, with the winners installed.
    entries = [dict(N=b["N"], K=b["K"], m_lo=b["m_lo"], m_hi=b["m_hi"], **b["chosen"]) for b in buckets]
    sg_set_table_override(entries)
    per_m = measure(GATE_MS, 20, device)
    sg_set_table_override([])
    table = {
        "generated_by": "python -m bf16_skinny_gemm_02_amd.tune",
        "device": f"{torch.cuda.get_device_name(device)} "
                  f"({torch.cuda.get_device_properties(device).gcnArchName})",
        "date": time.strftime("%Y-%m-%d"),
        "margin": MARGIN,
        "timing": f"hipGraph of R calls over R weight copies (>= 512 MiB, at most {MAX_COPIES}), "
                  f"median of 3 x {args.reps} replays, µs per call",
        "buckets": buckets,
        "overlap": {"per_m": per_m, "max_tokens": derive_gate(per_m)},
    }
    emit(table, args.out_dir)
    log(f"[tune] wrote {len(buckets)} entries, gate {table['overlap']['max_tokens']}, "
        f"{time.time() - t0:.0f} s")


if __name__ == "__main__":
    main()
