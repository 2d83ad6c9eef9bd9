"""Every configuration the tuner can time, through skinny_gemm's explicit
config, against the oracle (MI355X).

The tuner installs candidates the library's support predicate accepts and
times them through the entry points; the chosen ones become the compiled
table.  Each such candidate must therefore compute the same result as the
rule's own choice: here every candidate of tune.candidates for a spread of
shapes (ragged N and K, one and several K-ranges, every kernel kind) runs with
a residual and is compared with the oracle, and the table's chosen
configurations run at the shapes they serve.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bf16_skinny_gemm_02_amd as sg
import oracle
import synth
from bf16_skinny_gemm_02_amd import tune
from tests.gpu_util import assert_close, dev, host, nan_like

pytestmark = pytest.mark.gpu

CASES = [(1, 1030, 2048), (1, 136, 7168), (3, 700, 2056), (8, 5200, 1000), (12, 2000, 1032),
         (16, 300, 4104), (24, 520, 1032), (40, 300, 2056), (64, 1000, 520), (100, 200, 1032),
         (256, 130, 264)]


def _bucket(M):
    return next((lo, hi) for lo, hi in tune.BUCKETS if lo <= M <= hi)


@pytest.mark.parametrize("M,N,K", CASES)
def test_every_candidate_matches_the_oracle(device, M, N, K):
    A, W, R = synth.gemm_inputs(M, N, K, seed=4400 + M + N + K, residual=True)
    ex, _ = oracle.gemm(A, W, R)
    Ad, Wd, Rd = dev(A, device), dev(W, device), dev(R, device)
    lo, hi = _bucket(M)
    ran = 0
    for c in tune.candidates(N, K, lo, hi):
        cfg = tune._full(c, M, N)
        if not sg.sg_config_supported(cfg, M, N, K):
            continue
        print(f"candidate M={M} N={N} K={K} cfg={cfg}", flush=True)
        out = nan_like((M, N), device)
        sg.skinny_gemm(Ad, Wd, Rd, out=out, cfg=cfg)
        torch.cuda.synchronize()
        assert_close(host(out), ex, f"{M}x{N}x{K} {cfg}")
        ran += 1
    assert ran >= 1


def test_table_configurations_at_their_shapes(device):
    """Each compiled entry at both ends of its range, on its own (N, K); the
    oracle computes 96 sampled output columns (first and last included; a
    column depends only on its own weight row)."""
    for e in sg.sg_tuned_table():
        for M in sorted({e["m_lo"], e["m_hi"]}):
            N, K = e["N"], e["K"]
            print(f"table entry M={M} N={N} K={K} {e}", flush=True)
            A, W, _ = synth.gemm_inputs(M, N, K, seed=4500 + M + N)
            out = nan_like((M, N), device)
            sg.skinny_gemm(dev(A, device), dev(W, device), out=out)
            torch.cuda.synchronize()
            rng = np.random.default_rng(M + N)
            cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 94)]))
            ex, _ = oracle.gemm(A, W[cols], None)
            assert_close(host(out)[:, cols], ex, f"table {M}x{N}x{K}")
