"""Benchmark of the KDA decode projections and the latent-MoE tail on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One step is one pass of the whole hot path over the decode batch sizes
M in {1, 2, 3, 4, 8, 16, 17, 32, 64}: for every M, the KDA projection (Q/K/V/G
and F_A/beta -> F_B) through kda_projection_fused, and the latent-MoE tail
(RMSNorm -> up-projection -> shared add) through latent_moe_tail_fused (at
17 <= M <= 64 its up-projection sums its two K splits inside the launch).  At
1 <= M <= 16 the projection is one
launch (the wave-split Q/K/V/G tile with a helper wave per workgroup that runs
the F_A/beta -> F_B chain); elsewhere it is the one-stream schedule of
kda_projection_overlap (the overlap gate is closed, its measured setting on
MI355X): the Q/K/V/G and F_A/beta rows as two segments of one launch, then F_B.
Each (op, M) is a hipGraph of R back-to-back calls that cycle through R copies
of the weights, with R chosen so that the copies span >= 512 MiB: the 256 MiB
Infinity Cache cannot hold them, so the weights stream from HBM on every call.
Inputs are resident in HBM before timing starts.

Reported ``value``: mean microseconds per KDA projection call over the M sweep
(the metric's unit).  Within each timed step the projection graphs of the
whole sweep run back to back between two events, then the tail graphs between
the next two: ``value`` is the projection half's time over its calls,
``tail_us_per_call`` the tail half's.

``roofline`` is the headline path's own unit of work: one projection call at
M = 8 (its one launch), that M's graph replayed back to back right after the
timed region between HIP events on its stream; ``traffic`` is that call's HBM
bytes from rocprofv3 counters; ``sweep_gbs`` the timed region's own rate.

After the timed region: the per-M ``breakdown`` (projection and tail µs, GB/s,
fractions of the HBM and MFMA peaks), and ``configs``, one entry per workload
of the benchmark's definition: the single GEMV (M = 1), the F_A/beta -> F_B
branch alone (two launches, and the one-launch entry point, under graph
replay and launched eagerly), the Q/K/V/G projection alone over the sweep,
the projection's schedules (one launch, one stream, two streams) against a
packed GEMM followed by F_B, and the
latent-MoE tail up to M = 256.  ``--comparators`` adds the vendor library on
the same work (torch.mm / addmm, i.e. hipBLASLt, with the RMSNorm in unfused
torch ops).  ``cpu_baseline``: the CPU oracle on this host, on all its threads
and on one.
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
        # kda_projection_fused's workspace: zero-filled once (its header), then reused.
        self.ws_one = torch.zeros(sg.sg_kda_workspace_bytes(sg.SG_KDA_ONE_LAUNCH, M, K, N_QKVG, N_AB),
                                  dtype=torch.uint8, device=device)
        self.aux, self.fork, self.join = aux, fork, join

    def call(self, r, schedule="fused"):
        """schedule: "fused" (kda_projection_fused: one launch where it fits,
        else the one-stream schedule), "one_stream" or "two_stream"
        (kda_projection_overlap)."""
        if schedule == "fused":
            sg.kda_projection_fused(self.x, self.packed[r], self.w_b[r], qkvg=self.qkvg, g1=self.g1,
                                    beta=self.beta, workspace=self.ws_one)
            return
        sg.kda_projection_overlap(self.x, self.packed[r], self.w_b[r], qkvg=self.qkvg, g1=self.g1,
                                  beta=self.beta, ws_main=self.ws_main, ws_aux=self.ws_aux,
                                  aux_stream=self.aux if schedule == "two_stream" else None,
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
        # latent_moe_tail_fused's workspace: zero-filled once (its header), then reused.
        self.ws = torch.zeros(sg.sg_workspace_bytes(sg.SG_OP_LATENT_TAIL_FUSED, M, D_HID, D_LAT),
                              dtype=torch.uint8, device=device)

    def call(self, r):
        sg.latent_moe_tail_fused(self.L, self.gamma, self.w_up[r], self.S, eps=1e-6, out=self.out,
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


# ---- roofline leg and counters -------------------------------------------------------

BREAKDOWN_REPS = 20
BREAKDOWN_REPEATS = 5   # per-M breakdown: median, and the lowest / highest repeat (p10 / p90 of 5)

ROOFLINE_M = 8   # the projection call the roofline leg times (one launch at 1 <= M <= 16)

# HBM traffic of one projection call at M = ROOFLINE_M (its one launch) from two rocprofv3
# --pmc runs of `bench.py --counters` (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 KiB per dispatch;
# factors from a 256 MiB device copy), summarised with the commands in
# profiles/kda_projection_and_tail_pmc_traffic.md.  Valid only for the sources it was measured on:
# any change to them reports traffic as null until the counters are taken again.
TRAFFIC_SOURCES = ("bf16_skinny_gemm_02_amd/csrc/mfma.hip", "bf16_skinny_gemm_02_amd/csrc/gemv.hip",
                   "bf16_skinny_gemm_02_amd/csrc/smallk.hip", "bf16_skinny_gemm_02_amd/csrc/sg_device.h",
                   "bf16_skinny_gemm_02_amd/csrc/sg_help.h", "bf16_skinny_gemm_02_amd/csrc/sg_fused.h",
                   "bf16_skinny_gemm_02_amd/csrc/dispatch.cpp", "bf16_skinny_gemm_02_amd/csrc/abi.cpp",
                   "bf16_skinny_gemm_02_amd/csrc/tuned_table.inc")
TRAFFIC_PMC = {"sources_sha256": "14b6eeb13f43906ceaae7fc958a3535114d1d1a171670fbc73ebf36a1024df21", "bytes_per_call": 62781725}


def sources_sha256():
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        h.update((ROOT / rel).read_bytes())
    return h.hexdigest()


def measured_traffic():
    if TRAFFIC_PMC["sources_sha256"] != sources_sha256():
        return None
    return TRAFFIC_PMC["bytes_per_call"]


COPY_BYTES = 256 << 20   # calibration copy: reads and writes exactly this many bytes
COUNTER_PROJ_M = (8, 64)
COUNTER_TAIL_M = (1, 8, 64, 256)


def counters_mode(device):
    """One eager pass for the PMC runs: three device-to-device copies of
    COPY_BYTES (their FETCH_SIZE / WRITE_SIZE per dispatch calibrate the
    counters against known traffic), then the projection call at M = 8 and
    64 and the latent-MoE tail at M = 1, 8, 64, 256, once per cold weight
    copy, twice over.  Prints what was launched and exits."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=device)
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    launched = {}
    for M in COUNTER_PROJ_M:
        c = ProjectionCase(M, device, None, None, None)
        for _ in range(2):
            for r in range(c.R):
                c.call(r)
        torch.cuda.synchronize()
        launched[f"projection_m{M}"] = {"calls": 2 * c.R, "bytes_per_call": proj_bytes(M),
                                        "one_launch": bool(sg.sg_kda_one_launch_fits(M, K, N_QKVG, N_AB, RANK, N_B)),
                                        "flops_per_call": proj_flops(M),
                                        "q": sg.sg_kda_select(sg.SG_KDA_QKVG, M, K, N_QKVG, N_AB),
                                        "f": sg.sg_kda_select(sg.SG_KDA_FAB, M, K, N_QKVG, N_AB)}
        del c
    for M in COUNTER_TAIL_M:
        c = TailCase(M, device)
        for _ in range(2):
            for r in range(c.R):
                c.call(r)
        torch.cuda.synchronize()
        launched[f"tail_m{M}"] = {"calls": 2 * c.R, "bytes_per_call": tail_bytes(M),
                                  "flops_per_call": tail_flops(M),
                                  "cfg": sg.sg_select(M, D_HID, D_LAT, True)}
        del c
    print(json.dumps({"copy_bytes": COPY_BYTES, "sources_sha256": sources_sha256(),
                      "launched": launched}), flush=True)


# ---- the benchmark's other workloads ---------------------------------------------------

def graph_us(fn, R, stream, reps=10, repeats=3):
    """Median over `repeats` of the mean µs per call of a graph of fn(0..R-1)."""
    g = capture(fn, R, stream)
    ts = sorted(time_graph(g, stream, reps) * 1000.0 / R for _ in range(repeats))
    del g
    return ts[len(ts) // 2]


def eager_us(fn, R, stream, reps=5, repeats=3):
    """Median over `repeats` of the mean µs per call of fn(0..R-1) launched one
    by one from the host (no graph), timed with events on `stream`."""
    ts = []
    with torch.cuda.stream(stream):
        for r in range(R):
            fn(r)
        for _ in range(repeats):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                for r in range(R):
                    fn(r)
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1000.0 / (reps * R))
    ts.sort()
    return ts[len(ts) // 2]


def fab_bytes(M):
    return 2 * (N_AB * K + N_B * RANK + M * K + M * ((N_AB - RANK) + N_B))


def config_fab_fb(device, stream, Ms=(1, 2, 4, 8)):
    """The F_A/beta -> F_B branch alone: kda_fab_fb_proj (two launches) and
    kda_fab_fb_proj_fused (one launch), as graphs over cold weight copies and
    launched eagerly from the host."""
    out = {}
    for M in Ms:
        x, w_ab, w_b = synth.fab_fb_inputs(M)
        R = copies_for(2 * (N_AB * K + N_B * RANK))
        xd = bf16_dev(x, device)
        a0, b0 = bf16_dev(w_ab, device), bf16_dev(w_b, device)
        was = [a0] + [a0.clone() for _ in range(R - 1)]
        wbs = [b0] + [b0.clone() for _ in range(R - 1)]
        g1 = torch.empty((M, N_B), dtype=torch.bfloat16, device=device)
        beta = torch.empty((M, N_AB - RANK), dtype=torch.bfloat16, device=device)
        ws = torch.zeros(sg.sg_workspace_bytes(sg.SG_OP_FAB_FB, M, N_AB, K), dtype=torch.uint8,
                         device=device)
        row = {}
        for name, fn in (("two_launch", sg.kda_fab_fb_proj), ("one_launch", sg.kda_fab_fb_proj_fused)):
            call = (lambda r, fn=fn: fn(xd, was[r], wbs[r], g1=g1, beta=beta, workspace=ws))
            row[f"{name}_graph_us"] = round(graph_us(call, R, stream), 3)
            row[f"{name}_eager_us"] = round(eager_us(call, min(R, 64), stream), 3)
        row["bytes"] = fab_bytes(M)
        row["two_launch_graph_gbs"] = round(fab_bytes(M) / (row["two_launch_graph_us"] * 1e-6) / 1e9, 1)
        out[str(M)] = row
        del was, wbs
    return out


def config_qkvg(device, stream, Ms=M_SWEEP):
    """The packed Q/K/V/G projection alone (kda_qkvg_proj) over the sweep."""
    out = {}
    for M in Ms:
        x, w = synth.qkvg_inputs(M)
        R = copies_for(2 * N_QKVG * K)
        xd = bf16_dev(x, device)
        w0 = bf16_dev(w, device)
        ws = [w0] + [w0.clone() for _ in range(R - 1)]
        o = torch.empty((M, N_QKVG), dtype=torch.bfloat16, device=device)
        wsp = torch.empty(max(sg.sg_workspace_bytes(sg.SG_OP_GEMM, M, N_QKVG, K), 256),
                          dtype=torch.uint8, device=device)
        us = graph_us(lambda r: sg.kda_qkvg_proj(xd, ws[r], out=o, workspace=wsp), R, stream,
                      reps=BREAKDOWN_REPS)
        cfg = sg.sg_select(M, N_QKVG, K)
        out[str(M)] = {"us": round(us, 3), "gbs": round(qkvg_bytes(M) / (us * 1e-6) / 1e9, 1),
                       "hbm_frac": round(qkvg_bytes(M) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                       "mfma_frac": round(2 * M * N_QKVG * K / (us * 1e-6) / 1e12 /
                                          MFMA_BF16_PEAK_TFLOPS, 4),
                       "kind": cfg["kind"], "grid": cfg["grid"], "k_split": cfg["k_split"]}
        del ws
    return out


def config_schedules(proj, device, stream, Ms=(1, 4, 8, 16, 32)):
    """The projection's schedules (one launch where it fits; one stream;
    fork/join onto an aux stream) and a plain packed GEMM over [W_qkvg; W_ab]
    followed by a second GEMM for F_B, all as graphs over the same cold weight
    copies."""
    out = {}
    for M in Ms:
        c = proj[M]
        fused = graph_us(lambda r, c=c: c.call(r, "fused"), c.R, stream)
        one = graph_us(lambda r, c=c: c.call(r, "one_stream"), c.R, stream)
        two = graph_us(lambda r, c=c: c.call(r, "two_stream"), c.R, stream)
        out_packed = torch.empty((M, N_QKVG + N_AB), dtype=torch.bfloat16, device=device)
        g1_s2 = torch.empty((M, N_B), dtype=torch.bfloat16, device=device)
        ws2 = torch.empty(max(sg.sg_workspace_bytes(sg.SG_OP_GEMM, M, N_QKVG + N_AB, K), 256),
                          dtype=torch.uint8, device=device)

        def s2_call(r, c=c):
            sg.skinny_gemm(c.x, c.packed[r], out=out_packed, workspace=ws2)
            sg.skinny_gemm(out_packed[:, N_QKVG:N_QKVG + RANK], c.w_b[r], out=g1_s2)

        s2 = graph_us(s2_call, c.R, stream)
        out[str(M)] = {"fused_us": round(fused, 3),
                       "fused_is_one_launch": bool(sg.sg_kda_one_launch_fits(M, K, N_QKVG, N_AB, RANK, N_B)),
                       "one_stream_us": round(one, 3), "two_stream_us": round(two, 3),
                       "packed_gemm_then_fb_us": round(s2, 3),
                       "one_launch_speedup_vs_one_stream": round(one / fused, 3),
                       "two_stream_speedup_vs_one_stream": round(one / two, 3),
                       "two_stream_speedup_vs_packed": round(s2 / two, 3),
                       "gate_picks": "two_stream" if sg.sg_overlap_gate(M, True, True, True, True)
                       else "one_stream"}
    return out


def config_tail(tail, device, stream, extra_Ms=(256,)):
    """The latent-MoE tail at the benchmark's batch sizes M = 1, 8, 64, 256
    (the sweep's cases plus the larger ones)."""
    out = {}
    for M in (1, 8, 64) + tuple(extra_Ms):
        c = tail[M] if M in tail else TailCase(M, device)
        us = graph_us(c.call, c.R, stream, reps=BREAKDOWN_REPS)
        cfg = sg.sg_select(M, D_HID, D_LAT, True)
        out[str(M)] = {"us": round(us, 3), "gbs": round(tail_bytes(M) / (us * 1e-6) / 1e9, 1),
                       "hbm_frac": round(tail_bytes(M) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                       "mfma_frac": round(tail_flops(M) / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                       "roofline_frac": round(roofline_time_us(tail_bytes(M), tail_flops(M)) / us, 4),
                       "kind": cfg["kind"], "grid": cfg["grid"], "k_split": cfg["k_split"]}
        if M not in tail:
            del c
    return out


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

def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def _oracle_rate(threads, budget_s):
    """Whole passes over the projection M sweep with the oracle on `threads`
    OpenMP threads, as many as fit in budget_s (at least one)."""
    import oracle
    oracle.set_threads(threads)
    inputs = {M: synth.overlap_inputs(M) for M in M_SWEEP}
    calls = passes = 0
    t0 = time.perf_counter()
    while True:
        for M in M_SWEEP:
            x, packed, w_b = inputs[M]
            oracle.projection_overlap(x, packed, w_b)
            calls += 1
        passes += 1
        if time.perf_counter() - t0 >= budget_s or passes >= 50:
            break
    dt = time.perf_counter() - t0
    return dt / calls * 1e6, calls, passes, dt


def cpu_baseline(budget_s=15.0):
    """The oracle (fp64, OpenMP over outputs) on this host, on a bounded
    sample: whole passes over the M sweep of the KDA projection, on all the
    host's threads, then on one."""
    cores = len(os.sched_getaffinity(0))
    cores = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
    cpu = _cpu_model()
    us, calls, passes, dt = _oracle_rate(cores, budget_s)
    us1, calls1, passes1, dt1 = _oracle_rate(1, budget_s)
    return {"value": us, "unit": "us/call", "cores": cores, "kind": "oracle",
            "sample": f"{passes} pass(es) over the KDA projection M sweep {M_SWEEP} "
                      f"({calls} calls, {dt:.1f} s, fp64 oracle, OpenMP {cores} threads, {cpu})",
            "single_thread": {"value": us1, "unit": "us/call", "cores": 1,
                              "sample": f"{passes1} pass(es), {calls1} calls, {dt1:.1f} s"}}


# ---- main -----------------------------------------------------------------------------

KINDS = {sg.SG_KIND_GEMV_ROW: "gemv_kernel", sg.SG_KIND_GEMV_SPLITK: "gemv_kernel",
         sg.SG_KIND_MFMA_WAVESPLIT: "wsplit_kernel", sg.SG_KIND_MFMA_TILE: "tile_kernel",
         sg.SG_KIND_MFMA_BLOCK: "block_kernel"}


def projection_kernels(M):
    if sg.sg_kda_one_launch_fits(M, K, N_QKVG, N_AB, RANK, N_B):
        return (f"wsplit_help_kernel, one launch: {N_QKVG // 16} wave-split workgroups of 16 "
                f"Q/K/V/G rows, each with a helper wave (F_A/beta producer units, then F_B hosts)")
    q = sg.sg_kda_select(sg.SG_KDA_QKVG, M, K, N_QKVG, N_AB)
    f = sg.sg_kda_select(sg.SG_KDA_FAB, M, K, N_QKVG, N_AB)
    return (f"{KINDS.get(q['kind'], '?')} with the Q/K/V/G and F_A/beta rows as two segments "
            f"({q['grid'] + f['grid']} workgroups), then fab_fb_tail_kernel (F_B"
            f"{' and the Q/K/V/G split-K reduction' if q['k_split'] > 1 else ''})")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload configs (the timed sweep and breakdown only)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--comparators", action="store_true",
                    help="also time the same work through torch (hipBLASLt) with an unfused RMSNorm")
    ap.add_argument("--counters", action="store_true",
                    help="counter-collection mode for rocprofv3 --pmc: a plain device copy of "
                         "known size (calibration), then the projection and the tail launched "
                         "eagerly over their cold weight copies; prints what ran and exits")
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
    sched = {M: "two_stream" if gate[M] else "fused" for M in M_SWEEP}
    g_proj = {M: capture(lambda r, c=proj[M], s=sched[M]: c.call(r, s), proj[M].R,
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
            "schedule": ("two_stream" if gate[M] else
                         "one_launch" if sg.sg_kda_one_launch_fits(M, K, N_QKVG, N_AB, RANK, N_B)
                         else "one_stream"),
        }
    # Every projection graph holds the same number of calls, so this is also
    # the mean over the sweep of the per-M time per call.
    value = t_proj_all * 1000.0 / calls_proj
    tail_value = t_tail_all * 1000.0 / calls_tail
    ms_per_step = wall * 1000.0 / args.steps

    # Roofline leg: the same M = ROOFLINE_M projection graph replayed back to
    # back right after the timed region, between two events on its stream.
    roof_reps = 100
    us_call = time_graph(g_proj[ROOFLINE_M], main_stream, roof_reps) * 1000.0 / proj[ROOFLINE_M].R
    achieved = proj_bytes(ROOFLINE_M) / (us_call * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "kernel": f"KDA projection call at M = {ROOFLINE_M}: {projection_kernels(ROOFLINE_M)}",
                "unit_of_work": "one call of the headline path",
                "us_per_call": round(us_call, 3),
                "algorithmic_bytes_per_call": proj_bytes(ROOFLINE_M),
                "calls_timed": roof_reps * proj[ROOFLINE_M].R,
                "sweep_gbs": round(sum(proj_bytes(M) for M in M_SWEEP) * args.steps * proj[1].R /
                                   (t_proj_all * 1e-3) / 1e9, 1)}
    roofline["sweep_frac"] = round(roofline["sweep_gbs"] / HBM_PEAK_GBS, 4)

    configs = {}
    if not args.no_configs:
        print("[bench] per-workload configs", file=sys.stderr, flush=True)
        q1 = config_qkvg(device, main_stream)
        configs["qkvg_gemv_m1"] = {"workload": "single bf16 GEMV x[1,7168] W[4096,7168]",
                                   **q1["1"]}
        configs["fab_fb"] = config_fab_fb(device, main_stream)
        configs["qkvg_sweep"] = q1
        configs["projection_schedules"] = config_schedules(proj, device, main_stream)
        configs["latent_tail"] = config_tail(tail, device, main_stream)

    if args.comparators:
        for M in M_SWEEP:
            c = proj[M]
            out_t = torch.empty((M, N_QKVG + N_AB), dtype=torch.bfloat16, device=device)
            g1_t = torch.empty((M, N_B), dtype=torch.bfloat16, device=device)

            def blas_proj(r, c=c, out_t=out_t, g1_t=g1_t):
                torch.mm(c.x, c.packed[r].t(), out=out_t)
                torch.mm(out_t[:, N_QKVG:N_QKVG + RANK], c.w_b[r].t(), out=g1_t)

            tc = tail[M]
            out_tt = torch.empty((M, D_HID), dtype=torch.bfloat16, device=device)

            def blas_tail(r, tc=tc, out_tt=out_tt):
                lf = tc.L.float()
                n = (lf * torch.rsqrt(lf.pow(2).mean(-1, keepdim=True) + 1e-6) *
                     tc.gamma.float()).to(torch.bfloat16)
                torch.addmm(tc.S, n, tc.w_up[r].t(), out=out_tt)

            b = breakdown[str(M)]
            b["torch_blas_projection_us"] = round(graph_us(blas_proj, c.R, main_stream), 3)
            b["torch_blas_tail_us"] = round(graph_us(blas_tail, tc.R, main_stream), 3)

    context = context_figures(device, main_stream)

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
            "description": "KDA projection per M through kda_projection_fused (one launch at "
                           "1 <= M <= 16, else the one-stream schedule the closed overlap gate picks; QKVG "
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
        "configs": configs,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
