"""Python face of the CPU oracle (oracle.c), plus the compositions built from it.

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the bench).

Every function takes and returns numpy arrays of bf16 bit patterns (uint16) and,
where useful, the unrounded float64 values.  Definitions and the passages they
follow (vLLM pull-request summaries on prhub.com.cn):

O1 ``gemm``          C = bf16(A @ W^T + R), fp64 sum, one rounding.
                     "Kimi K3 support, phase 1" (#50089), _skinny_gemm.py,
                     CuteSkinnyGemm docstring and its residual epilogue.
O2 ``qkvg``          O1 with the packed q,k,v,g rows of one TP8 rank, no residual.
                     "Overlap low-M TP8 KDA projections" (#54697),
                     low_latency_gemm.py run_qkvg.
O3 ``fab_fb``        P = bf16(x @ W_ab^T); f_a = P[:, :rank]; beta = P[:, rank:];
                     g1 = bf16(f_a @ W_b^T) with f_a already bf16.
                     #54697, low_latency_gemm.py run_fab_fb (split into f_a and
                     beta, the bf16 f_a tensor feeds the F_B GEMM).
O4 ``projection_overlap``  (O2 on packed rows [0, n_qkvg), O3 on the next n_ab
                     rows): #54697 run_kda_projection_overlap, and the packed
                     sequential fallback in kda.py forward.
O5 ``latent_tail``   r = 1/sqrt(mean(L^2) + eps); n = bf16(L*r*gamma);
                     out = bf16(S + n @ W_up^T).
                     #50089, latent_moe_runner.py LatentMoERunner docstring.
                     variant 1 (default): the RMSNorm output n is a bf16 tensor
                     fed to the up-projection, as in the runner's unfused path.
                     variant 0 keeps n in fp64 (used to bound the drift
                     between the two readings).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB = _HERE / "liboracle.so"

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> Path:
    """Compile oracle.c into liboracle.so (gcc -O2, OpenMP, no fast-math)."""
    if force or not _LIB.exists():
        tmp = _LIB.with_suffix(".so.tmp")
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists():
            build()
        lib = ctypes.CDLL(str(_LIB))
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_gemm.restype = None
        lib.oracle_gemm.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    _u16p, ctypes.c_long, _u16p, ctypes.c_long,
                                    _u16p, ctypes.c_long, _f64p, _u16p, ctypes.c_long]
        lib.oracle_rms_scale.restype = None
        lib.oracle_rms_scale.argtypes = [ctypes.c_int, ctypes.c_int, _u16p, ctypes.c_long,
                                         ctypes.c_double, _f64p]
        lib.oracle_latent_tail.restype = None
        lib.oracle_latent_tail.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           _u16p, _u16p, ctypes.c_double, _u16p, _u16p,
                                           ctypes.c_int, _f64p, _u16p]
        _lib = lib
    return _lib


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return a


def _p16(a):
    return None if a is None else a.ctypes.data_as(_u16p)


def _p64(a):
    return a.ctypes.data_as(_f64p)


def round_bf16(values) -> np.ndarray:
    """float64 values -> bf16 bits, round to nearest, ties to even (oracle.c)."""
    lib = _load()
    v = np.asarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    flat_in = v.reshape(-1)
    flat_out = out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.oracle_round_bf16(float(flat_in[i]))
    return out


def to_f64(bits) -> np.ndarray:
    """bf16 bits -> float64, exact."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm(A: np.ndarray, W: np.ndarray, R: np.ndarray | None = None):
    """O1: returns (exact float64 [M,N], bf16 bits [M,N])."""
    A = _u16(A)
    W = _u16(W)
    M, K = A.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    if R is not None:
        R = _u16(R)
        if R.shape != (M, N):
            raise ValueError("residual shape")
    exact = np.zeros((M, N), dtype=np.float64)
    bits = np.zeros((M, N), dtype=np.uint16)
    if M and N:
        _load().oracle_gemm(M, N, K, _p16(A), K, _p16(W), K, _p16(R), N,
                            _p64(exact), _p16(bits), N)
    return exact, bits


def qkvg(x: np.ndarray, w_qkvg: np.ndarray):
    """O2: the packed Q/K/V/G projection."""
    return gemm(x, w_qkvg)


def fab_fb(x: np.ndarray, w_ab: np.ndarray, w_b: np.ndarray, rank: int = 128):
    """O3: returns dict with p (exact, bits), f_a, beta, g1 (exact, bits)."""
    p_exact, p_bits = gemm(x, w_ab)
    f_a = np.ascontiguousarray(p_bits[:, :rank])
    beta = np.ascontiguousarray(p_bits[:, rank:])
    g1_exact, g1_bits = gemm(f_a, w_b)
    return {"p_exact": p_exact, "p_bits": p_bits, "f_a": f_a, "beta": beta,
            "beta_exact": p_exact[:, rank:], "g1_exact": g1_exact, "g1_bits": g1_bits}


def projection_overlap(x, packed, w_b, n_qkvg: int = 4096, n_ab: int = 136, rank: int = 128):
    """O4: (qkvg on packed[:n_qkvg], fab_fb on packed[n_qkvg:n_qkvg+n_ab])."""
    packed = _u16(packed)
    q_exact, q_bits = gemm(x, packed[:n_qkvg])
    fb = fab_fb(x, packed[n_qkvg:n_qkvg + n_ab], w_b, rank)
    return {"qkvg_exact": q_exact, "qkvg_bits": q_bits, **fb}


def rms_scale(L: np.ndarray, eps: float) -> np.ndarray:
    L = _u16(L)
    M, d = L.shape
    r = np.zeros(M, dtype=np.float64)
    if M:
        _load().oracle_rms_scale(M, d, _p16(L), d, float(eps), _p64(r))
    return r


def latent_tail(L, gamma, eps, w_up, S=None, variant: int = 1):
    """O5: returns (exact float64 [M,D], bf16 bits [M,D])."""
    L = _u16(L)
    gamma = _u16(gamma)
    w_up = _u16(w_up)
    M, d = L.shape
    D, d2 = w_up.shape
    if d2 != d or gamma.shape != (d,):
        raise ValueError("latent / gamma / w_up shapes")
    if S is not None:
        S = _u16(S)
        if S.shape != (M, D):
            raise ValueError("shared shape")
    exact = np.zeros((M, D), dtype=np.float64)
    bits = np.zeros((M, D), dtype=np.uint16)
    if M and D:
        _load().oracle_latent_tail(M, d, D, _p16(L), _p16(gamma), float(eps), _p16(w_up),
                                   _p16(S), int(variant), _p64(exact), _p16(bits))
    return exact, bits


def set_threads(n: int) -> None:
    """OpenMP threads for the oracle's output loop (used by the CPU baseline)."""
    os.environ["OMP_NUM_THREADS"] = str(int(n))
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(ctypes.c_int(int(n)))
    except OSError:
        pass
