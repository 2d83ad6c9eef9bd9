"""Pins for the CPU oracle (runs on any host).

Each test ties the oracle to something other than itself: hand-derived rounding
cases, a library routine (torch's float32 -> bf16 conversion), exact rational
brute force on small inputs, the integer lattice, identity / zero / one-hot
weights, closed forms of RMSNorm, and algebraic invariants.  The last tests
plant plausible mistakes in copies of the oracle's results and check that the
pins reject them.
"""
from __future__ import annotations

import math
import random
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import exact

GOLDEN = Path(__file__).resolve().parent / "golden"


# ---- rounding -------------------------------------------------------------------

def _golden_rne():
    rows = []
    for line in (GOLDEN / "bf16_rne_cases.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        expr, bits, why = (s.strip() for s in line.split("|", 2))
        rows.append((expr, int(bits, 16), why))
    return rows


@pytest.mark.parametrize("expr,bits,why", _golden_rne())
def test_round_bf16_golden(expr, bits, why):
    value = eval(expr, {"float": float})  # fixture expressions are plain arithmetic
    assert int(oracle.round_bf16([value])[0]) == bits, why


def test_round_bf16_nan():
    b = int(oracle.round_bf16([float("nan")])[0])
    assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0


def test_round_bf16_matches_torch_on_float32():
    """float32 inputs: torch's float32 -> bf16 cast is a single RNE step."""
    rng = np.random.default_rng(7)
    bits32 = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    # finite only; include every tie pattern (low half == 0x8000) of some values
    ties = (rng.integers(0, 2 ** 16, size=4000).astype(np.uint32) << 16) | 0x8000
    allbits = np.concatenate([bits32, ties.astype(np.uint32)])
    vals = allbits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(vals.astype(np.float64))
    mism = np.nonzero(ref != got)[0]
    assert mism.size == 0, [(float(vals[i]), hex(ref[i]), hex(got[i])) for i in mism[:5]]


def test_round_bf16_matches_exact_search():
    """Doubles with bits below float32 precision: compare with the exact search."""
    rnd = random.Random(3)
    vals = []
    for _ in range(3000):
        e = rnd.randint(-140, 127)
        vals.append(rnd.choice([-1, 1]) * rnd.random() * 2.0 ** e)
    got = oracle.round_bf16(vals)
    for v, g in zip(vals, got):
        want, _ = exact.nearest_bf16(exact.Fraction(v))
        assert int(g) == want, (v, hex(g), hex(want))


def test_widening_is_exact():
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    f = oracle.to_f64(bits)
    back = (f.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(back, bits)


# ---- O1 gemm ------------------------------------------------------------------------

def _random_bits(rng, shape, scale=1.0):
    return synth.to_bf16_bits(rng.normal(0, scale, size=shape))


@pytest.mark.parametrize("M,N,K,res", [(1, 1, 8, False), (3, 5, 8, True), (4, 7, 16, False),
                                       (2, 3, 24, True), (5, 2, 40, True), (8, 8, 8, False)])
def test_gemm_bruteforce_exact(M, N, K, res):
    rng = np.random.default_rng(1000 + M * 100 + N * 10 + K)
    A = _random_bits(rng, (M, K))
    W = _random_bits(rng, (N, K), 0.3)
    R = _random_bits(rng, (M, N)) if res else None
    ex, bits = oracle.gemm(A, W, R)
    for m in range(M):
        for n in range(N):
            v = exact.exact_dot(A[m], W[n])
            if R is not None:
                v += exact.bits_to_fraction(R[m, n])
            # the fp64 sum is within ~K ulp(double) of the exact sum
            assert abs(exact.Fraction(ex[m, n]) - v) <= abs(v) * 1e-14 + 1e-300
            want, _ = exact.nearest_bf16(v)
            if exact.tie_distance(v) > abs(v) * 1e-12:
                assert int(bits[m, n]) == want, (m, n, float(v))


def test_gemm_lattice_full_k():
    """x in {-2..2}, W in {-1,0,1}/64: every partial sum is exact in fp64."""
    M, N, K = 3, 24, 7168
    x = synth.lattice_activation((M, K), seed=11)
    w = synth.lattice_weight((N, K), seed=12)
    ex, bits = oracle.gemm(x, w)
    xi = np.rint(oracle.to_f64(x)).astype(np.int64)
    wi = np.rint(oracle.to_f64(w) * 64).astype(np.int64)
    s = xi @ wi.T
    assert np.array_equal(ex, s / 64.0)
    for m in range(M):
        for n in range(N):
            want, _ = exact.nearest_bf16(exact.Fraction(int(s[m, n]), 64))
            assert int(bits[m, n]) == want


def test_gemm_identity_and_one_hot():
    rng = np.random.default_rng(5)
    M, K = 4, 64
    x = _random_bits(rng, (M, K))
    eye = synth.to_bf16_bits(np.eye(K))
    _, bits = oracle.gemm(x, eye)
    assert np.array_equal(bits, x)
    # one-hot rows pick arbitrary columns
    cols = rng.integers(0, K, size=10)
    oh = np.zeros((10, K))
    oh[np.arange(10), cols] = 1.0
    _, bits = oracle.gemm(x, synth.to_bf16_bits(oh))
    assert np.array_equal(bits, x[:, cols])


def test_gemm_zero_weights_gives_residual():
    rng = np.random.default_rng(6)
    M, N, K = 3, 17, 32
    x = _random_bits(rng, (M, K))
    R = synth.to_bf16_bits(np.abs(rng.normal(size=(M, N))) + 0.5)
    _, bits = oracle.gemm(x, np.zeros((N, K), np.uint16), R)
    assert np.array_equal(bits, R)
    _, bits = oracle.gemm(x, np.zeros((N, K), np.uint16))
    assert not bits.any()


def test_gemm_linearity_and_scaling():
    rng = np.random.default_rng(8)
    M, N, K = 2, 9, 512
    xi = rng.integers(-8, 9, size=(M, K)).astype(np.float64)
    yi = rng.integers(-8, 9, size=(M, K)).astype(np.float64)
    W = _random_bits(rng, (N, K), 0.05)
    ex_x, _ = oracle.gemm(synth.to_bf16_bits(xi), W)
    ex_y, _ = oracle.gemm(synth.to_bf16_bits(yi), W)
    ex_xy, _ = oracle.gemm(synth.to_bf16_bits(xi + yi), W)
    assert np.allclose(ex_xy, ex_x + ex_y, rtol=1e-12, atol=1e-12)
    ex_2x, _ = oracle.gemm(synth.to_bf16_bits(4.0 * xi), W)
    assert np.array_equal(ex_2x, 4.0 * ex_x)


def test_gemm_concatenation_and_symmetry():
    rng = np.random.default_rng(9)
    M, K = 3, 96
    x = _random_bits(rng, (M, K))
    W1 = _random_bits(rng, (7, K), 0.1)
    W2 = _random_bits(rng, (5, K), 0.1)
    _, b_cat = oracle.gemm(x, np.concatenate([W1, W2]))
    _, b1 = oracle.gemm(x, W1)
    _, b2 = oracle.gemm(x, W2)
    assert np.array_equal(b_cat, np.concatenate([b1, b2], axis=1))
    ex_t, _ = oracle.gemm(W1, x)
    ex, _ = oracle.gemm(x, W1)
    assert np.allclose(ex_t.T, ex, rtol=1e-13, atol=0)


def test_gemm_output_statistics():
    """x ~ N(0,1), W ~ N(0,1/K): outputs have unit variance (scaling sanity)."""
    x, w = synth.qkvg_inputs(1, seed=42, N=1024)
    ex, _ = oracle.gemm(x, w)
    assert 0.9 < float(np.std(ex)) < 1.1


# ---- O3 F_A/beta -> F_B ---------------------------------------------------------------

def test_fab_fb_bruteforce_small():
    rng = np.random.default_rng(21)
    M, K, n_ab, rank, n_b = 2, 32, 12, 8, 6
    x = _random_bits(rng, (M, K))
    w_ab = _random_bits(rng, (n_ab, K), 0.2)
    w_b = _random_bits(rng, (n_b, rank), 0.3)
    out = oracle.fab_fb(x, w_ab, w_b, rank)
    P = np.zeros((M, n_ab), np.uint16)
    for m in range(M):
        for j in range(n_ab):
            P[m, j], _ = exact.nearest_bf16(exact.exact_dot(x[m], w_ab[j]))
    assert np.array_equal(out["f_a"], P[:, :rank])
    assert np.array_equal(out["beta"], P[:, rank:])
    for m in range(M):
        for i in range(n_b):
            v = exact.exact_dot(P[m, :rank], w_b[i])  # F_B consumes the bf16 f_a
            if exact.tie_distance(v) > abs(v) * 1e-12:
                assert int(out["g1_bits"][m, i]) == exact.nearest_bf16(v)[0]


def test_fab_fb_rounds_f_a_before_f_b():
    """g1 is computed from the bf16 f_a, not the fp64 one (differs somewhere)."""
    x, w_ab, w_b = synth.fab_fb_inputs(4)
    out = oracle.fab_fb(x, w_ab, w_b)
    g1_from_exact = out["p_exact"][:, :128] @ oracle.to_f64(w_b).T
    assert not np.array_equal(out["g1_exact"], g1_from_exact)
    assert np.allclose(out["g1_exact"], g1_from_exact, rtol=0, atol=5e-2)


def test_projection_overlap_matches_packed_gemm():
    x, packed, w_b = synth.overlap_inputs(2, K=512, n_qkvg=64, n_ab=20, rank=16, n_b=32)
    o = oracle.projection_overlap(x, packed, w_b, n_qkvg=64, n_ab=20, rank=16)
    _, packed_bits = oracle.gemm(x, packed)
    assert np.array_equal(o["qkvg_bits"], packed_bits[:, :64])
    assert np.array_equal(o["p_bits"], packed_bits[:, 64:84])
    assert np.array_equal(o["beta"], packed_bits[:, 80:84])


# ---- O5 latent-MoE tail -----------------------------------------------------------------

def _one_hot_rows(D, d, cols):
    w = np.zeros((D, d))
    w[np.arange(D), cols] = 1.0
    return synth.to_bf16_bits(w)


def test_rms_scale_closed_forms():
    d, eps = 2048, 1e-6
    c = 1.5
    L = synth.to_bf16_bits(np.full((1, d), c))
    r = oracle.rms_scale(L, eps)[0]
    assert abs(r - 1.0 / math.sqrt(c * c + eps)) <= 1e-15
    L = np.zeros((1, d), np.uint16)
    L[0, 17] = synth.to_bf16_bits(np.array([c]))[0]
    r = oracle.rms_scale(L, eps)[0]
    assert abs(r - 1.0 / math.sqrt(c * c / d + eps)) <= 1e-15


def test_latent_tail_constant_and_one_hot_rows():
    d, D, eps = 2048, 24, 1e-6
    rng = np.random.default_rng(31)
    gamma = synth.uniform((d,), 0.5, 1.5, seed=31, tensor_id=synth.T_GAMMA)
    g = oracle.to_f64(gamma)
    cols = rng.integers(0, d, size=D)
    w_up = _one_hot_rows(D, d, cols)
    c = -0.75
    L = synth.to_bf16_bits(np.full((1, d), c))
    ex, _ = oracle.latent_tail(L, gamma, eps, w_up, variant=0)
    want = c / math.sqrt(c * c + eps) * g[cols]
    assert np.allclose(ex[0], want, rtol=1e-14, atol=0)
    # variant 1: each output is the bf16 rounding of c * r * gamma_k itself
    _, bits = oracle.latent_tail(L, gamma, eps, w_up)
    r = 1.0 / math.sqrt(c * c + eps)
    for j, k in enumerate(cols):
        assert int(bits[0, j]) == exact.nearest_bf16(exact.Fraction(c * r * float(g[k])))[0]
    # one-hot latent row: n_j = gamma_j * c / sqrt(c^2/d + eps), about +-45.25 gamma_j
    j = int(cols[3])
    L = np.zeros((1, d), np.uint16)
    L[0, j] = synth.to_bf16_bits(np.array([c]))[0]
    ex, _ = oracle.latent_tail(L, gamma, eps, w_up, variant=0)
    expect = np.where(cols == j, g[j] * c / math.sqrt(c * c / d + eps), 0.0)
    assert np.allclose(ex[0], expect, rtol=1e-14, atol=0)
    assert abs(abs(expect[3]) / g[j] - math.sqrt(d)) < 0.1  # ~45.25 for |c| >> sqrt(eps*d)


def test_latent_tail_zero_weights_and_unit_rows():
    rng = np.random.default_rng(32)
    M, d, D = 3, 256, 40
    L, gamma, w_up, S = synth.tail_inputs(M, seed=77, d=d, D=D)
    _, bits = oracle.latent_tail(L, gamma, 1e-6, np.zeros((D, d), np.uint16), S)
    assert np.array_equal(bits, S)
    # rows of +-1, gamma = 1, eps = 0: r = 1 exactly and the tail reduces to O1
    Lpm = synth.to_bf16_bits(rng.choice([-1.0, 1.0], size=(M, d)))
    ones = synth.to_bf16_bits(np.ones(d))
    _, t_bits = oracle.latent_tail(Lpm, ones, 0.0, w_up, S)
    _, g_bits = oracle.gemm(Lpm, w_up, S)
    assert np.array_equal(t_bits, g_bits)


def test_latent_tail_scale_invariance_and_variants():
    M, d, D = 4, 2048, 64
    L, gamma, w_up, S = synth.tail_inputs(M, seed=78, D=D)
    ex, _ = oracle.latent_tail(L, gamma, 1e-6, w_up, S, variant=0)
    L4 = synth.to_bf16_bits(oracle.to_f64(L) * 4.0)  # exact power-of-two scaling
    ex4, _ = oracle.latent_tail(L4, gamma, 1e-6, w_up, S, variant=0)
    assert np.allclose(ex4, ex, rtol=0, atol=1e-5 * np.abs(ex).max())
    # Rounding the normalised latent to bf16 perturbs each product by <= 2^-9
    # relative; over 2048 terms of unit-variance products the output moves by
    # ~1e-3 (one sigma).
    ex1, _ = oracle.latent_tail(L, gamma, 1e-6, w_up, S, variant=1)
    assert np.all(np.abs(ex1 - ex) <= 5e-3 * np.maximum(1.0, np.abs(ex)))
    assert np.abs(ex1 - ex).max() > 1e-4  # the two readings do differ


def test_latent_tail_variant_drift_at_full_size():
    """The drift between the two readings of the RMSNorm output on the tail
    workload at its largest batch (M = 256, d = 2048, D = 7168, the inputs
    the GPU tests use): one sigma ~1.0e-3 and a maximum of 7.9e-3 scaled by
    max(1, |out|), below the 1e-2 budget but close to it, which is why the
    GPU is held to one reading (the bf16 normalised latent) rather than
    either."""
    L, gamma, w_up, S = synth.tail_inputs(256)
    ex0, _ = oracle.latent_tail(L, gamma, 1e-6, w_up, S, variant=0)
    ex1, _ = oracle.latent_tail(L, gamma, 1e-6, w_up, S, variant=1)
    diff = np.abs(ex1 - ex0)
    scaled = diff / np.maximum(1.0, np.abs(ex0))
    assert 7.0e-3 < scaled.max() < 8.5e-3, scaled.max()
    assert 0.8e-3 < diff.std() < 1.3e-3, diff.std()


# ---- planted mistakes: the pins above must reject each ------------------------------------

def test_pins_reject_planted_mistakes():
    rng = np.random.default_rng(41)
    M, N, K = 3, 5, 16
    A = _random_bits(rng, (M, K))
    W = _random_bits(rng, (N, K), 0.3)
    R = _random_bits(rng, (M, N))

    def brute(A, W, R):
        out = np.zeros((A.shape[0], W.shape[0]), np.uint16)
        for m in range(A.shape[0]):
            for n in range(W.shape[0]):
                v = exact.exact_dot(A[m], W[n]) + (exact.bits_to_fraction(R[m, n]) if R is not None else 0)
                out[m, n] = exact.nearest_bf16(v)[0]
        return out

    truth = brute(A, W, R)
    assert np.array_equal(oracle.gemm(A, W, R)[1], truth)
    # 1. dropped last k term
    assert not np.array_equal(oracle.gemm(A[:, :-8], W[:, :-8], R)[1], truth)
    # 2. residual omitted
    assert not np.array_equal(oracle.gemm(A, W)[1], truth)
    # 3. operand order / index swap (W rows reversed)
    assert not np.array_equal(oracle.gemm(A, W[::-1].copy(), R)[1], truth)
    # 4. sign flip of the weights
    assert not np.array_equal(oracle.gemm(A, W ^ np.uint16(0x8000), R)[1], truth)
    # 5. truncation instead of round-to-nearest-even
    ex, _ = oracle.gemm(A, W, R)
    trunc = (ex.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert not np.array_equal(trunc, truth) or np.array_equal(oracle.round_bf16(ex), truth)
