"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only DRAWS inputs; it holds none of the arithmetic of the method.
Values are drawn in float64 from numpy's PCG64 generator, narrowed to float32 by
numpy and to bf16 by torch's float32 -> bfloat16 conversion (round to nearest
even), and handed out as uint16 bf16 bit patterns, so that the CPU oracle and
the GPU path read exactly the same bits.

Distributions follow the decode workloads of the Kimi-K3 KDA projections and the
latent-MoE tail: activations ~ N(0, 1), weights ~ N(0, 1/K) (unit-variance
outputs), RMSNorm gamma ~ U(0.5, 1.5).  The real model weights are not
available; these Gaussian stand-ins have the same shapes.

Seeds: every tensor gets its own stream, ``PCG64([seed, tensor_id])``; a
workload's seed is ``1000 * workload_id + M``.
"""
from __future__ import annotations

import numpy as np
import torch

# Shapes of one TP8 rank's slice of Kimi-K3 (hidden size 7168).
HIDDEN = 7168          # K of every KDA projection
N_QKVG = 4096          # q, k, v, g: 8 heads x 128 dims each
N_AB = 136             # f_a (rank 128) + 8 beta heads
RANK = 128             # F_A low rank = K of F_B
N_B = 1024             # F_B output (g1)
D_LATENT = 2048        # latent-MoE latent width
D_HIDDEN = 7168        # latent-MoE up-projection output

# Workload ids used in seeds.
WL_QKVG_GEMV = 1
WL_FAB_FB = 2
WL_QKVG_SWEEP = 3
WL_OVERLAP = 4
WL_LATENT_TAIL = 5

# Tensor ids (second word of the seed).
T_X, T_W, T_WAB, T_WB, T_L, T_GAMMA, T_WUP, T_S, T_R = range(9)


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), int(tensor_id)]))


def to_bf16_bits(values: np.ndarray) -> np.ndarray:
    """float array -> uint16 bf16 bit patterns (float32 first, then RNE to bf16)."""
    f32 = np.ascontiguousarray(np.asarray(values, dtype=np.float32))
    t = torch.from_numpy(f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact widening)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def gaussian(shape, std: float, seed: int, tensor_id: int) -> np.ndarray:
    return to_bf16_bits(_rng(seed, tensor_id).normal(0.0, std, size=shape))


def uniform(shape, lo: float, hi: float, seed: int, tensor_id: int) -> np.ndarray:
    return to_bf16_bits(_rng(seed, tensor_id).uniform(lo, hi, size=shape))


def lattice_activation(shape, seed: int, tensor_id: int = T_X) -> np.ndarray:
    """Integers in {-2..2}: exact in bf16."""
    return to_bf16_bits(_rng(seed, tensor_id).integers(-2, 3, size=shape).astype(np.float64))


def lattice_weight(shape, seed: int, tensor_id: int = T_W) -> np.ndarray:
    """{-1, 0, 1} * 2^-6: exact in bf16."""
    v = _rng(seed, tensor_id).integers(-1, 2, size=shape).astype(np.float64)
    return to_bf16_bits(v * 2.0 ** -6)


def gemm_inputs(M: int, N: int, K: int, seed: int, residual: bool = False):
    """x ~ N(0,1) [M,K], W ~ N(0,1/K) [N,K], optional residual ~ N(0,1) [M,N]."""
    x = gaussian((M, K), 1.0, seed, T_X)
    w = gaussian((N, K), (1.0 / max(K, 1)) ** 0.5, seed, T_W)
    r = gaussian((M, N), 1.0, seed, T_R) if residual else None
    return x, w, r


def qkvg_inputs(M: int, seed: int | None = None, K: int = HIDDEN, N: int = N_QKVG):
    seed = 1000 * WL_QKVG_SWEEP + M if seed is None else seed
    x, w, _ = gemm_inputs(M, N, K, seed)
    return x, w


def fab_fb_inputs(M: int, seed: int | None = None, K: int = HIDDEN, n_ab: int = N_AB,
                  rank: int = RANK, n_b: int = N_B):
    """x [M,K] ~ N(0,1); W_ab [n_ab,K] ~ N(0,1/K); W_b [n_b,rank] ~ N(0,1/rank)."""
    seed = 1000 * WL_FAB_FB + M if seed is None else seed
    x = gaussian((M, K), 1.0, seed, T_X)
    w_ab = gaussian((n_ab, K), (1.0 / K) ** 0.5, seed, T_WAB)
    w_b = gaussian((n_b, rank), (1.0 / rank) ** 0.5, seed, T_WB)
    return x, w_ab, w_b


def overlap_inputs(M: int, seed: int | None = None, K: int = HIDDEN, n_qkvg: int = N_QKVG,
                   n_ab: int = N_AB, rank: int = RANK, n_b: int = N_B):
    """x, packed [W_qkvg; W_ab] [n_qkvg+n_ab, K], W_b."""
    seed = 1000 * WL_OVERLAP + M if seed is None else seed
    x = gaussian((M, K), 1.0, seed, T_X)
    w_qkvg = gaussian((n_qkvg, K), (1.0 / K) ** 0.5, seed, T_W)
    w_ab = gaussian((n_ab, K), (1.0 / K) ** 0.5, seed, T_WAB)
    w_b = gaussian((n_b, rank), (1.0 / rank) ** 0.5, seed, T_WB)
    packed = np.concatenate([w_qkvg, w_ab], axis=0)
    return x, packed, w_b


def tail_inputs(M: int, seed: int | None = None, d: int = D_LATENT, D: int = D_HIDDEN):
    """L [M,d] ~ N(0,1); gamma [d] ~ U(0.5,1.5); W_up [D,d] ~ N(0,1/d); S [M,D] ~ N(0,1)."""
    seed = 1000 * WL_LATENT_TAIL + M if seed is None else seed
    L = gaussian((M, d), 1.0, seed, T_L)
    gamma = uniform((d,), 0.5, 1.5, seed, T_GAMMA)
    w_up = gaussian((D, d), (1.0 / d) ** 0.5, seed, T_WUP)
    S = gaussian((M, D), 1.0, seed, T_S)
    return L, gamma, w_up, S
