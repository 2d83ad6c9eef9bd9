"""Benchmark of the KDA decode projections and the latent-MoE tail on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One step is one pass of the whole hot path over the decode batch sizes
M in {1, 2, 3, 4, 8, 16, 17, 32, 64}: for every M, the KDA projection (Q/K/V/G
and F_A/beta -> F_B) in the schedule the overlap gate picks for that M, and the
latent-MoE tail (RMSNorm -> up-projection -> shared add).  With the gate
closed (its measured setting on MI355X) the projection runs on one stream: the
Q/K/V/G and F_A/beta rows as two segments of one launch, then F_B.
Each (op, M) is a hipGraph of R back-to-back calls that cycle through R copies
of the weights, with R chosen so that the copies span >= 512 MiB: the 256 MiB
Infinity Cache cannot hold them, so the weights stream from HBM on every call.
Inputs are resident in HBM before timing starts.

Reported ``value``: mean microseconds per KDA projection call over the M sweep
(the metric's unit).  Within each timed step the projection graphs of the
whole sweep run back to back between two events, then the tail graphs between
the next two: ``value`` is the projection half's time over its calls,
``tail_us_per_call`` the tail half's.  The per-M ``breakdown`` (projection and
tail µs, GB/s, fraction of HBM peak) is measured after the timed region, each
graph replayed back to back.  ``--comparators`` adds, per M, the forced
two-stream schedule (fork/join events, F_A/beta -> F_B on an aux stream), the
forced single-stream schedule, a plain packed GEMM followed by a second GEMM
for F_B, and the vendor library on the same work (torch.mm / addmm, i.e.
hipBLASLt, with the RMSNorm in unfused torch ops).  The line also carries the
roofline of the dominant kernel (the wave-split MFMA tile at M = 8, with the
M = 1 GEMV beside it, each timed with HIP events on its own stream) and the
CPU oracle timed on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from pathlib import Path

import numpy as np
import torch

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

import bf16_skinny_gemm_02_amd as sg  # noqa: E402
import synth  # noqa: E402

METRIC = "µs/call and % of HBM roofline (GB/s) for KDA decode projections, M=1..64"
M_SWEEP = [1, 2, 3, 4, 8, 16, 17, 32, 64]
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
COLD_BYTES = 512 << 20          # weights rotated across at least this many bytes

K = synth.HIDDEN
N_QKVG, N_AB, RANK, N_B = synth.N_QKVG, synth.N_AB, synth.RANK, synth.N_B
D_LAT, D_HID = synth.D_LATENT, synth.D_HIDDEN


def bf16_dev(bits, device):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).to(device).view(
        torch.bfloat16)


# ---- algorithmic bytes / flops (each weight, input and output touched once) --------

def proj_bytes(M):
    return 2 * ((N_QKVG + N_AB) * K + N_B * RANK + M * K + M * (N_QKVG + (N_AB - RANK) + N_B))


def proj_flops(M):
    return 2 * M * ((N_QKVG + N_AB) * K + N_B * RANK)


def qkvg_bytes(M):
    return 2 * (N_QKVG * K + M * K + M * N_QKVG)


def tail_bytes(M):
    return 2 * (D_HID * D_LAT + M * D_LAT + D_LAT + 2 * M * D_HID)


def tail_flops(M):
    return 2 * M * D_HID * D_LAT


def roofline_time_us(nbytes, flops):
    """Time at the binding roofline: the larger of the HBM and the MFMA bound."""
    return max(nbytes / (HBM_PEAK_GBS * 1e3), flops / (MFMA_BF16_PEAK_TFLOPS * 1e6))


# ---- graph construction -------------------------------------------------------------

def copies_for(weight_bytes):
    return max(2, math.ceil(COLD_BYTES / weight_bytes))


class ProjectionCase:
    """R KDA projection calls at batch M, one weight copy each."""

    def __init__(self, M, device, aux, fork, join):
        x, packed, w_b = synth.overlap_inputs(M)
        self.M = M
        self.R = copies_for(2 * ((N_QKVG + N_AB) * K + N_B * RANK))
        self.x = bf16_dev(x, device)
        p0 = bf16_dev(packed, device)
        b0 = bf16_dev(w_b, device)
        self.packed = [p0] + [p0.clone() for _ in range(self.R - 1)]
        self.w_b = [b0] + [b0.clone() for _ in range(self.R - 1)]
        self.qkvg = torch.empty((M, N_QKVG), dtype=torch.bfloat16, device=device)
        self.g1 = torch.empty((M, N_B), dtype=torch.bfloat16, device=device)
        self.beta = torch.empty((M, N_AB - RANK), dtype=torch.bfloat16, device=device)
        self.ws_aux = torch.zeros(max(sg.sg_kda_workspace_bytes(1, M, K, N_QKVG, N_AB), 256),
                                  dtype=torch.uint8, device=device)
        self.ws_main = torch.zeros(max(sg.sg_kda_workspace_bytes(0, M, K, N_QKVG, N_AB), 256),
                                   dtype=torch.uint8, device=device)
        self.aux, self.fork, self.join = aux, fork, join

    def call(self, r, concurrent=True):
        sg.kda_projection_overlap(self.x, self.packed[r], self.w_b[r], qkvg=self.qkvg, g1=self.g1,
                                  beta=self.beta, ws_main=self.ws_main, ws_aux=self.ws_aux,
                                  aux_stream=self.aux if concurrent else None,
                                  fork=self.fork, join=self.join)


class TailCase:
    def __init__(self, M, device):
        L, gamma, w_up, S = synth.tail_inputs(M)
        self.M = M
        self.R = copies_for(2 * D_HID * D_LAT)
        self.L = bf16_dev(L, device)
        self.gamma = bf16_dev(gamma, device)
        w0 = bf16_dev(w_up, device)
        self.w_up = [w0] + [w0.clone() for _ in range(self.R - 1)]
        self.S = bf16_dev(S, device)
        self.out = torch.empty((M, D_HID), dtype=torch.bfloat16, device=device)
        self.ws = torch.empty(max(sg.sg_workspace_bytes(sg.SG_OP_LATENT_TAIL, M, D_HID, D_LAT), 256),
                              dtype=torch.uint8, device=device)

    def call(self, r):
        sg.latent_moe_tail(self.L, self.gamma, self.w_up[r], self.S, eps=1e-6, out=self.out,
                           workspace=self.ws)


def capture(fn, R, stream):
    """hipGraph of fn(0), ..., fn(R-1) captured on `stream`."""
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for r in range(R):       # warm the code paths once outside capture
            fn(r)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in range(R):
                fn(r)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    return g


def time_graph(g, stream, reps, warm=3):
    """Mean ms per replay, timed with events on the replay stream.  `warm`
    untimed replays go first: the GPU is busy (and at its working clocks)
    when the start event is reached, and the host's submission of the first
    timed replay is not counted."""
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for _ in range(warm):
            g.replay()
        start.record(stream)
        for _ in range(reps):
            g.replay()
        stop.record(stream)
    stop.synchronize()
    return start.elapsed_time(stop) / reps


# ---- dominant-kernel roofline leg ---------------------------------------------------

BREAKDOWN_REPS = 20
BREAKDOWN_REPEATS = 5   # per-M breakdown: median, and the lowest / highest repeat (p10 / p90 of 5)

ROOFLINE_M = 8   # the wave-split MFMA tile serves M = 2..16, five of the nine sweep points

# HBM traffic of the roofline kernel from two rocprofv3 --pmc runs of `bench.py --counters`
# (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 KiB per dispatch; factors from a 256 MiB device copy),
# summarised with the commands in profiles/qkvg_wsplit_m8_pmc_traffic.md.  Valid only for the
# kernel sources it was measured on: any change to them reports traffic as null until the
# counters are taken again.
TRAFFIC_SOURCES = ("bf16_skinny_gemm_02_amd/csrc/mfma.hip", "bf16_skinny_gemm_02_amd/csrc/sg_device.h",
                   "bf16_skinny_gemm_02_amd/csrc/dispatch.cpp")
TRAFFIC_PMC = {"sources_sha256": "ff8c56fa576d1e4e66bc76e381eda24c5571d6f976ddabb910e38533ef6e01b4",
               "bytes_per_launch": 59784527}


def measured_traffic():
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        h.update((ROOT / rel).read_bytes())
    return TRAFFIC_PMC["bytes_per_launch"] if h.hexdigest() == TRAFFIC_PMC["sources_sha256"] else None


def qkvg_kernel_leg(device, M, reps=200):
    """Average duration of the Q/K/V/G projection kernel at batch M
    (x[M,7168] x W[4096,7168]^T, one launch per call for M <= 16), back-to-back
    launches on one stream cycling cold weight copies, timed with HIP events
    recorded on that stream."""
    x, w = synth.qkvg_inputs(M, seed=1000 * synth.WL_QKVG_SWEEP + M)
    R = copies_for(2 * N_QKVG * K)
    xd = bf16_dev(x, device)
    w0 = bf16_dev(w, device)
    ws = [w0] + [w0.clone() for _ in range(R - 1)]
    out = torch.empty((M, N_QKVG), dtype=torch.bfloat16, device=device)
    stream = torch.cuda.Stream(device)
    g = capture(lambda r: sg.kda_qkvg_proj(xd, ws[r], out=out), R, stream)
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    ms = time_graph(g, stream, reps)
    us = ms * 1000.0 / R
    gbs = qkvg_bytes(M) / (us * 1e-6) / 1e9
    cfg = sg.sg_select(M, N_QKVG, K)
    kinds = {sg.SG_KIND_GEMV_ROW: "gemv_kernel", sg.SG_KIND_MFMA_WAVESPLIT: "wsplit_kernel",
             sg.SG_KIND_MFMA_TILE: "tile_kernel", sg.SG_KIND_MFMA_BLOCK: "block_kernel"}
    name = f"{kinds.get(cfg['kind'], '?')} (kda_qkvg_proj M={M}, {cfg['grid']} workgroups)"
    return {"kernel": name, "us_per_launch": us, "launches_timed": reps * R, "gbs": gbs,
            "bytes": qkvg_bytes(M)}


COPY_BYTES = 256 << 20   # calibration copy: reads and writes exactly this many bytes


def counters_mode(device):
    """One eager pass for the PMC runs: three device-to-device copies of
    COPY_BYTES (their FETCH_SIZE / WRITE_SIZE per dispatch calibrate the
    counters against known traffic), then the roofline kernel once per cold
    weight copy, twice over."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=device)
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    M = ROOFLINE_M
    x, w = synth.qkvg_inputs(M, seed=1000 * synth.WL_QKVG_SWEEP + M)
    R = copies_for(2 * N_QKVG * K)
    xd = bf16_dev(x, device)
    w0 = bf16_dev(w, device)
    ws = [w0] + [w0.clone() for _ in range(R - 1)]
    out = torch.empty((M, N_QKVG), dtype=torch.bfloat16, device=device)
    for _ in range(2):
        for r in range(R):
            sg.kda_qkvg_proj(xd, ws[r], out=out)
    torch.cuda.synchronize()
    del ws
    # The MFMA tile paths, once each, for the matrix-core counters: the packed
    # projection at M = 64 (128-row tiles) and the latent-MoE tail at M = 256
    # (block tile).
    pc = ProjectionCase(64, device, None, None, None)
    pc.call(0, concurrent=False)
    tc = TailCase(256, device)
    tc.call(0)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "roofline_m": M, "launches": 2 * R,
                      "algorithmic_bytes_per_launch": qkvg_bytes(M),
                      "mfma_legs": {"projection_m64_flops": proj_flops(64),
                                    "tail_m256_flops": tail_flops(256)}}), flush=True)


# ---- context: launch floor and a plain device copy ---------------------------------

def context_figures(device, stream):
    """The floor of one graph kernel node (a one-element add, 100 per graph)
    and the bandwidth of a plain 512 MiB device-to-device copy (bytes read +
    bytes written), the scale against which the projections' GB/s read."""
    t = torch.zeros(1, device=device)
    g = capture(lambda r: t.add_(1.0), 100, stream)
    floor = time_graph(g, stream, 20) * 1000.0 / 100
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device=device)
    src.fill_(1)
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        dst.copy_(src)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(5):
            dst.copy_(src)
        stop.record(stream)
    stop.synchronize()
    us = start.elapsed_time(stop) * 1000.0 / 5
    del src, dst
    return {"graph_kernel_node_floor_us": round(floor, 3),
            "copy_512MiB_gbs_read_plus_write": round(2 * n / (us * 1e-6) / 1e9, 1)}


# ---- CPU baseline -------------------------------------------------------------------

def cpu_baseline(budget_s=15.0):
    """The oracle (fp64, OpenMP over outputs) on this host's cores, on a bounded
    sample: whole passes over the M sweep of the KDA projection, as many as fit
    in the budget (at least one)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    cores = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
    oracle.set_threads(cores)
    inputs = {M: synth.overlap_inputs(M) for M in M_SWEEP}
    calls = 0
    t0 = time.perf_counter()
    passes = 0
    while True:
        for M in M_SWEEP:
            x, packed, w_b = inputs[M]
            oracle.projection_overlap(x, packed, w_b)
            calls += 1
        passes += 1
        if time.perf_counter() - t0 >= budget_s or passes >= 50:
            break
    dt = time.perf_counter() - t0
    cpu = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": dt / calls * 1e6, "unit": "us/call", "cores": cores, "kind": "oracle",
            "sample": f"{passes} pass(es) over the KDA projection M sweep {M_SWEEP} "
                      f"({calls} calls, {dt:.1f} s, fp64 oracle, OpenMP {cores} threads, {cpu})"}


# ---- main -----------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--comparators", action="store_true",
                    help="also time the forced two-stream and one-stream schedules, a plain "
                         "packed GEMM followed by F_B, and the same work through torch "
                         "(hipBLASLt) with an unfused RMSNorm")
    ap.add_argument("--counters", action="store_true",
                    help="counter-collection mode for rocprofv3 --pmc: a plain device copy of "
                         "known size (calibration), then the roofline kernel launched eagerly "
                         "over its cold weight copies; prints the byte counts and exits")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the hot path has no cross-GPU step (each TP8 rank's "
              "projection slice is independent), so only --gpus 1 is supported.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    if args.counters:
        counters_mode(device)
        return
    print(f"[bench] building cases for M in {M_SWEEP}", file=sys.stderr, flush=True)

    main_stream = torch.cuda.Stream(device)
    aux = torch.cuda.Stream(device)
    fork, join = sg.HipEvent(), sg.HipEvent()
    proj = {M: ProjectionCase(M, device, aux, fork, join) for M in M_SWEEP}
    tail = {M: TailCase(M, device) for M in M_SWEEP}
    gate = {M: sg.sg_overlap_gate(M, True, True, True, True) for M in M_SWEEP}
    g_proj = {M: capture(lambda r, c=proj[M], conc=gate[M]: c.call(r, concurrent=conc), proj[M].R,
                         main_stream) for M in M_SWEEP}
    g_tail = {M: capture(lambda r, c=tail[M]: c.call(r), tail[M].R, main_stream) for M in M_SWEEP}
    print("[bench] graphs captured", file=sys.stderr, flush=True)

    def step():
        for M in M_SWEEP:
            g_proj[M].replay()
            g_tail[M].replay()

    with torch.cuda.stream(main_stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps, synchronised on both sides.  Within
    # a step the projection graphs of the whole sweep run back to back, then
    # the tail graphs; three events on the replay stream split the step into
    # its two halves (an event between every graph would stall the stream at
    # each boundary).  They are read after the region.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    with torch.cuda.stream(main_stream):
        for st in range(args.steps):
            e = evs[st]
            e[0].record(main_stream)
            for M in M_SWEEP:
                g_proj[M].replay()
            e[1].record(main_stream)
            for M in M_SWEEP:
                g_tail[M].replay()
            e[2].record(main_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    t_proj_all = sum(e[0].elapsed_time(e[1]) for e in evs)
    t_tail_all = sum(e[1].elapsed_time(e[2]) for e in evs)
    calls_proj = args.steps * sum(proj[M].R for M in M_SWEEP)
    calls_tail = args.steps * sum(tail[M].R for M in M_SWEEP)
    print(f"[bench] timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    # Per-M breakdown (after the timed region): each graph replayed back to
    # back, timed with events on the replay stream.
    breakdown = {}
    for M in M_SWEEP:
        ps = sorted(time_graph(g_proj[M], main_stream, BREAKDOWN_REPS) * 1000.0 / proj[M].R
                    for _ in range(BREAKDOWN_REPEATS))
        ts = sorted(time_graph(g_tail[M], main_stream, BREAKDOWN_REPS) * 1000.0 / tail[M].R
                    for _ in range(BREAKDOWN_REPEATS))
        pu, tu = ps[len(ps) // 2], ts[len(ts) // 2]
        breakdown[str(M)] = {
            "proj_us": round(pu, 3),
            "proj_us_p10_p90": [round(ps[0], 3), round(ps[-1], 3)],
            "proj_gbs": round(proj_bytes(M) / (pu * 1e-6) / 1e9, 1),
            "proj_hbm_frac": round(proj_bytes(M) / (pu * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "proj_tflops": round(proj_flops(M) / (pu * 1e-6) / 1e12, 2),
            "proj_mfma_frac": round(proj_flops(M) / (pu * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "proj_roofline_frac": round(roofline_time_us(proj_bytes(M), proj_flops(M)) / pu, 4),
            "tail_us": round(tu, 3),
            "tail_us_p10_p90": [round(ts[0], 3), round(ts[-1], 3)],
            "tail_gbs": round(tail_bytes(M) / (tu * 1e-6) / 1e9, 1),
            "tail_hbm_frac": round(tail_bytes(M) / (tu * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "tail_tflops": round(tail_flops(M) / (tu * 1e-6) / 1e12, 2),
            "tail_mfma_frac": round(tail_flops(M) / (tu * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "tail_roofline_frac": round(roofline_time_us(tail_bytes(M), tail_flops(M)) / tu, 4),
            "weight_copies": [proj[M].R, tail[M].R],
            "schedule": "two_stream" if gate[M] else "one_stream",
        }
    # Every projection graph holds the same number of calls, so this is also
    # the mean over the sweep of the per-M time per call.
    value = t_proj_all * 1000.0 / calls_proj
    tail_value = t_tail_all * 1000.0 / calls_tail
    ms_per_step = wall * 1000.0 / args.steps

    if args.comparators:
        for M in M_SWEEP:
            c = proj[M]
            g_two = capture(lambda r, c=c: c.call(r, concurrent=True), c.R, main_stream)
            two = time_graph(g_two, main_stream, 10) * 1000.0 / c.R
            g_one = capture(lambda r, c=c: c.call(r, concurrent=False), c.R, main_stream)
            one = time_graph(g_one, main_stream, 10) * 1000.0 / c.R
            pw = c.packed
            out_packed = torch.empty((M, N_QKVG + N_AB), dtype=torch.bfloat16, device=device)
            g1_s2 = torch.empty((M, N_B), dtype=torch.bfloat16, device=device)
            ws2 = torch.empty(max(sg.sg_workspace_bytes(sg.SG_OP_GEMM, M, N_QKVG + N_AB, K), 256),
                              dtype=torch.uint8, device=device)

            def s2_call(r, c=c, out_packed=out_packed, g1_s2=g1_s2, ws2=ws2, pw=pw):
                sg.skinny_gemm(c.x, pw[r], out=out_packed, workspace=ws2)
                sg.skinny_gemm(out_packed[:, N_QKVG:N_QKVG + RANK], c.w_b[r], out=g1_s2)

            g_s2 = capture(s2_call, c.R, main_stream)
            s2 = time_graph(g_s2, main_stream, 10) * 1000.0 / c.R
            # The vendor library on the same work: torch.mm (hipBLASLt) over the packed
            # weight, then a second torch.mm for F_B on the bf16 f_a columns.
            out_t = torch.empty((M, N_QKVG + N_AB), dtype=torch.bfloat16, device=device)
            g1_t = torch.empty((M, N_B), dtype=torch.bfloat16, device=device)

            def blas_proj(r, c=c, out_t=out_t, g1_t=g1_t, pw=pw):
                torch.mm(c.x, pw[r].t(), out=out_t)
                torch.mm(out_t[:, N_QKVG:N_QKVG + RANK], c.w_b[r].t(), out=g1_t)

            g_bp = capture(blas_proj, c.R, main_stream)
            bp = time_graph(g_bp, main_stream, 10) * 1000.0 / c.R
            # ... and the unfused latent-MoE tail: RMSNorm in torch ops (fp32, bf16
            # result), then torch.addmm with the shared-expert partial.
            tc = tail[M]
            out_tt = torch.empty((M, D_HID), dtype=torch.bfloat16, device=device)

            def blas_tail(r, tc=tc, out_tt=out_tt):
                lf = tc.L.float()
                n = (lf * torch.rsqrt(lf.pow(2).mean(-1, keepdim=True) + 1e-6) *
                     tc.gamma.float()).to(torch.bfloat16)
                torch.addmm(tc.S, n, tc.w_up[r].t(), out=out_tt)

            g_bt = capture(blas_tail, tc.R, main_stream)
            bt = time_graph(g_bt, main_stream, 10) * 1000.0 / tc.R
            b = breakdown[str(M)]
            b["two_stream_us"] = round(two, 3)
            b["one_stream_us"] = round(one, 3)
            b["packed_gemm_then_fb_us"] = round(s2, 3)
            b["two_stream_speedup_vs_one_stream"] = round(one / two, 3)
            b["torch_blas_projection_us"] = round(bp, 3)
            b["torch_blas_tail_us"] = round(bt, 3)
            del g_two, g_one, g_s2, g_bp, g_bt

    context = context_figures(device, main_stream)
    leg = qkvg_kernel_leg(device, ROOFLINE_M)
    roofline = {"bound": "hbm", "achieved": round(leg["gbs"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(leg["gbs"] / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(),
                "kernel": leg["kernel"], "us_per_launch": round(leg["us_per_launch"], 3),
                "algorithmic_bytes_per_launch": leg["bytes"]}
    gemv = qkvg_kernel_leg(device, 1)
    roofline["gemv_m1"] = {"kernel": gemv["kernel"], "us_per_launch": round(gemv["us_per_launch"], 3),
                           "achieved": round(gemv["gbs"], 1),
                           "frac": round(gemv["gbs"] / HBM_PEAK_GBS, 4),
                           "algorithmic_bytes_per_launch": gemv["bytes"]}

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "kda_decode_projection_sweep",
            "description": "KDA projection per M in the schedule the overlap gate picks (QKVG "
                           "[4096,7168] and F_A/beta [136,7168] -> F_B [1024,128], hipGraph), "
                           "plus the latent-MoE tail (RMSNorm 2048 -> up-proj [7168,2048] + "
                           "shared add) per M; value = mean us per projection call over the "
                           "sweep; weights cold (rotated over >= 512 MiB)",
            "m_sweep": M_SWEEP, "hidden": K, "n_qkvg": N_QKVG, "n_ab": N_AB, "rank": RANK,
            "n_b": N_B, "d_latent": D_LAT, "d_hidden": D_HID, "parallelism": "single_gpu",
        },
        "roofline": roofline,
        "tail_us_per_call": round(tail_value, 3),
        "context": context,
        "breakdown": breakdown,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
