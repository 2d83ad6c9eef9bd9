"""Measure the overlap gate of the KDA projection on this GPU.

    python -m bf16_skinny_gemm_02_amd.tune_gate [--m 1,2,...,64] [--reps 20]

The two-branch KDA projection ("Overlap low-M TP8 KDA projections",
run_kda_projection_overlap) runs the Q/K/V/G rows on the main stream and
F_A/beta -> F_B on an auxiliary stream; the forward gate takes that schedule
for 0 < M <= KDA_PROJECTION_OVERLAP_MAX_TOKENS, a constant the pages set from
their own measurements.  This script makes the same measurement here: for
every M it times both schedules of ``kda_projection_overlap`` (the
single-stream one and the fork/join one), each as a hipGraph of back-to-back
calls over weight copies spanning >= 512 MiB (cold weights), and derives the
gate as the largest M such that the two-stream schedule is faster at every
M' <= M (0 when it never is).  It prints one JSON line with the per-M times,
the derived gate and the library's compiled value (``sg_overlap_max_tokens``);
the constant in the configuration table is set from this output.
"""
from __future__ import annotations

import argparse
import json
import math

import torch

from . import HipEvent, kda_projection_overlap, sg_kda_workspace_bytes, sg_overlap_max_tokens

HIDDEN, N_QKVG, N_AB, RANK, N_B = 7168, 4096, 136, 128, 1024
COLD_BYTES = 512 << 20


def _graph(fn, R, stream):
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for r in range(R):
            fn(r)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in range(R):
                fn(r)
    torch.cuda.synchronize()
    return g


def _time(g, stream, reps):
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for _ in range(3):
            g.replay()
        start.record(stream)
        for _ in range(reps):
            g.replay()
        stop.record(stream)
    stop.synchronize()
    return start.elapsed_time(stop) / reps


def measure(ms, reps, device):
    gen = torch.Generator(device="cpu").manual_seed(1234)
    weight_bytes = 2 * ((N_QKVG + N_AB) * HIDDEN + N_B * RANK)
    R = max(2, math.ceil(COLD_BYTES / weight_bytes))
    packed0 = (torch.randn(N_QKVG + N_AB, HIDDEN, generator=gen) / math.sqrt(HIDDEN)).to(torch.bfloat16)
    w_b0 = (torch.randn(N_B, RANK, generator=gen) / math.sqrt(RANK)).to(torch.bfloat16)
    packed = [packed0.to(device) for _ in range(R)]
    w_b = [w_b0.to(device) for _ in range(R)]
    stream = torch.cuda.Stream(device)
    aux = torch.cuda.Stream(device)
    fork, join = HipEvent(), HipEvent()
    rows = []
    for M in ms:
        x = torch.randn(M, HIDDEN, generator=gen).to(torch.bfloat16).to(device)
        qkvg = torch.empty(M, N_QKVG, dtype=torch.bfloat16, device=device)
        g1 = torch.empty(M, N_B, dtype=torch.bfloat16, device=device)
        beta = torch.empty(M, N_AB - RANK, dtype=torch.bfloat16, device=device)
        ws_main = torch.zeros(max(sg_kda_workspace_bytes(0, M, HIDDEN, N_QKVG, N_AB), 256),
                              dtype=torch.uint8, device=device)
        ws_aux = torch.zeros(max(sg_kda_workspace_bytes(1, M, HIDDEN, N_QKVG, N_AB), 256),
                             dtype=torch.uint8, device=device)

        def call(r, concurrent):
            kda_projection_overlap(x, packed[r], w_b[r], qkvg=qkvg, g1=g1, beta=beta,
                                   ws_main=ws_main, ws_aux=ws_aux,
                                   aux_stream=aux if concurrent else None, fork=fork, join=join)

        one = _time(_graph(lambda r: call(r, False), R, stream), stream, reps) * 1000.0 / R
        two = _time(_graph(lambda r: call(r, True), R, stream), stream, reps) * 1000.0 / R
        rows.append({"M": M, "one_stream_us": round(one, 3), "two_stream_us": round(two, 3)})
        print(f"[tune_gate] M={M} one-stream {one:.2f} us, two-stream {two:.2f} us", flush=True)
    return rows


def derive_gate(rows):
    """Largest M such that the two-stream schedule wins at every measured M' <= M."""
    gate = 0
    for row in sorted(rows, key=lambda r: r["M"]):
        if row["two_stream_us"] < row["one_stream_us"]:
            gate = row["M"]
        else:
            break
    return gate


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--m", default="1,2,3,4,6,8,10,12,14,16,24,32,48,64")
    ap.add_argument("--reps", type=int, default=20)
    args = ap.parse_args()
    if not torch.cuda.is_available():
        raise SystemExit("tune_gate needs a GPU")
    device = torch.device("cuda:0")
    ms = sorted({int(v) for v in args.m.split(",") if v.strip()})
    rows = measure(ms, args.reps, device)
    gate = derive_gate(rows)
    print(json.dumps({"overlap_max_tokens_measured": gate,
                      "overlap_max_tokens_compiled": sg_overlap_max_tokens(),
                      "per_m": rows}), flush=True)


if __name__ == "__main__":
    main()
