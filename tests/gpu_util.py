"""Helpers for the GPU parity tests: host <-> device transfer of bf16 bit
patterns and the tolerance check against the oracle."""
from __future__ import annotations

import numpy as np
import torch

# Tolerance for bf16 outputs against the fp64 oracle, per element:
# |gpu - oracle| <= 1e-2 * max(1, |oracle|).  The GPU's own error budget is one
# bf16 rounding (<= 2^-9 relative) plus fp32 accumulation (~1e-6 relative over
# 7168 terms) plus, in the latent tail, the bf16 rounding of the normalised
# operand (~1e-3 absolute, one sigma).
RTOL = 1e-2


def dev(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bits -> bf16 tensor on the device."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.to(device).view(torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bits on the host."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).copy()


def to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(
        np.float32).astype(np.float64)


def assert_close(gpu_bits: np.ndarray, oracle_exact: np.ndarray, what: str, rtol: float = RTOL):
    g = to_f64(gpu_bits)
    assert g.shape == oracle_exact.shape, (what, g.shape, oracle_exact.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output (unwritten element?)"
    err = np.abs(g - oracle_exact)
    bound = rtol * np.maximum(1.0, np.abs(oracle_exact))
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{what}: {len(bad)} elements out of tolerance, first "
                           f"{[tuple(i) for i in bad[:4]]}, max err {err.max():.3e}")
    return float(err.max())


def cosine(gpu_bits: np.ndarray, oracle_exact: np.ndarray) -> float:
    g = to_f64(gpu_bits).ravel()
    o = oracle_exact.ravel()
    return float(g @ o / (np.linalg.norm(g) * np.linalg.norm(o) + 1e-300))


def nan_like(shape, device) -> torch.Tensor:
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device=device)
