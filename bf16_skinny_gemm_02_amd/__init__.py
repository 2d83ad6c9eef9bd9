"""bf16 skinny GEMMs for the Kimi-K3 KDA decode projections and the latent-MoE
tail on AMD Instinct MI355X (gfx950).

Thin Python binding of libskinny_gemm.so (C ABI: include/skinny_gemm.h).  The
functions carry the C names and only marshal arguments: every step of the
computation runs in the library's HIP kernels.  PyTorch supplies device memory
and streams.  Tensors are bf16 (or int16 / uint16 bit-pattern views), on the
GPU, with unit stride along K.

Sources for what each call computes (vLLM pull-request summaries on
prhub.com.cn): "Kimi K3 support, phase 1" (#50089) -- CuteSkinnyGemm,
ShapeDynamicSkinnyGemm._config, LatentMoERunner; "Overlap low-M TP8 KDA
projections" (#54697) -- run_kda_projection_overlap, run_qkvg, run_fab_fb,
the KimiK3DeltaAttention.forward gate.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (SG_KIND_MFMA_BLOCK, SG_KIND_GEMV_ROW, SG_KIND_GEMV_SMALLK, SG_KIND_GEMV_SPLITK,  # noqa: F401
                   SG_KIND_MFMA_TILE, SG_KIND_MFMA_WAVESPLIT, SG_KIND_NONE,
                   SG_KDA_FAB, SG_KDA_FAB_ALONE, SG_KDA_ONE_LAUNCH, SG_KDA_QKVG, SG_OP_FAB_FB, SG_OP_GEMM,
                   SG_OP_LATENT_TAIL, SG_OP_LATENT_TAIL_FUSED, SgConfig, SgTableEntry)

__all__ = [
    "sg_select", "sg_overlap_gate", "sg_overlap_max_tokens", "sg_workspace_bytes",
    "sg_kda_select", "sg_kda_workspace_bytes", "sg_kda_one_launch_fits", "sg_version",
    "sg_config_supported",
    "sg_config_workspace_bytes", "sg_tuned_table", "sg_set_table_override",
    "skinny_gemm", "kda_qkvg_proj", "kda_fab_fb_proj", "kda_projection_overlap",
    "latent_moe_tail", "kda_projection_noalloc", "kda_fab_fb_proj_fused", "kda_projection_fused",
    "latent_moe_tail_fused", "HipEvent",
    "library_path",
]

_16BIT = (torch.bfloat16, torch.int16, torch.uint16)


def library_path() -> str:
    return str(_lib.LIB_PATH)


# ---- host-only queries ------------------------------------------------------

def sg_select(M: int, N: int, K: int, has_residual: bool = False) -> dict:
    """The configuration the library uses for an [M,K] x [N,K]^T problem."""
    cfg = SgConfig()
    _lib.check(_lib.load().sg_select(int(M), int(N), int(K), int(bool(has_residual)),
                                     ctypes.byref(cfg)), "sg_select")
    return cfg.as_dict()


def sg_overlap_gate(M: int, x_contiguous: bool, have_aux_stream: bool, have_events: bool,
                    enabled: bool = True) -> bool:
    return bool(_lib.load().sg_overlap_gate(int(M), int(bool(x_contiguous)),
                                            int(bool(have_aux_stream)), int(bool(have_events)),
                                            int(bool(enabled))))


def sg_overlap_max_tokens() -> int:
    return int(_lib.load().sg_overlap_max_tokens())


def sg_workspace_bytes(op: int, M: int, N: int, K: int) -> int:
    return int(_lib.load().sg_workspace_bytes(int(op), int(M), int(N), int(K)))


def sg_kda_select(which: int, M: int, K: int, n_qkvg: int, n_ab: int) -> dict:
    """The configuration a KDA projection entry point uses for one row range
    (SG_KDA_QKVG, SG_KDA_FAB: kda_projection_overlap; SG_KDA_FAB_ALONE:
    kda_fab_fb_proj)."""
    cfg = SgConfig()
    _lib.check(_lib.load().sg_kda_select(int(which), int(M), int(K), int(n_qkvg), int(n_ab),
                                         ctypes.byref(cfg)), "sg_kda_select")
    return cfg.as_dict()


def sg_kda_workspace_bytes(which: int, M: int, K: int, n_qkvg: int, n_ab: int) -> int:
    return int(_lib.load().sg_kda_workspace_bytes(int(which), int(M), int(K), int(n_qkvg),
                                                  int(n_ab)))


def sg_kda_one_launch_fits(M: int, K: int, n_qkvg: int, n_ab: int, rank: int, n_b: int) -> bool:
    """Whether kda_projection_fused runs these shapes as one launch."""
    return bool(_lib.load().sg_kda_one_launch_fits(int(M), int(K), int(n_qkvg), int(n_ab), int(rank),
                                                   int(n_b)))


def _config(cfg: dict) -> SgConfig:
    c = SgConfig()
    for name, _ in SgConfig._fields_:
        setattr(c, name, int(cfg.get(name, 1 if name == "nt_weights" else 0)))
    return c


def sg_config_supported(cfg: dict, M: int, N: int, K: int) -> bool:
    """Whether the kernels can run configuration `cfg` (a dict of sg_config_t
    fields) on an M x N x K problem."""
    st = _lib.load().sg_config_supported(ctypes.byref(_config(cfg)), int(M), int(N), int(K))
    if st == _lib.SG_ERR_INVALID_ARG:
        _lib.check(st, "sg_config_supported")
    return st == _lib.SG_OK


def sg_config_workspace_bytes(cfg: dict, M: int, N: int) -> int:
    return int(_lib.load().sg_config_workspace_bytes(ctypes.byref(_config(cfg)), int(M), int(N)))


def sg_tuned_table() -> list:
    """The compiled measured table, as a list of dicts (N, K, m_lo, m_hi,
    kind, rows, waves, k_unroll, k_split)."""
    ptr = ctypes.POINTER(SgTableEntry)()
    n = int(_lib.load().sg_tuned_table(ctypes.byref(ptr)))
    return [ptr[i].as_dict() for i in range(n)]


def sg_set_table_override(entries: list) -> None:
    """Replace the process-wide override table that sg_select consults first
    (an empty list clears it).  Not to be called while other calls are in
    flight or being captured."""
    arr = (SgTableEntry * max(1, len(entries)))()
    for i, e in enumerate(entries):
        for name in _lib.TABLE_FIELDS:
            setattr(arr[i], name, int(e[name]))
    _lib.check(_lib.load().sg_set_table_override(arr, len(entries)), "sg_set_table_override")


def sg_version() -> str:
    return _lib.load().sg_version().decode()


# ---- marshalling helpers ----------------------------------------------------

def _check_tensor(t: torch.Tensor, name: str, ndim: int, contiguous: bool = False,
                  on_gpu: bool = True) -> None:
    """Type, dtype, rank and layout first, the device last, so that layout
    errors are reported the same way on any host."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in _16BIT:
        raise TypeError(f"{name} must be bfloat16 (or a 16-bit bit-pattern view), got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if t.numel() and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dimension")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (the C ABI takes no row stride for it)")
    if on_gpu and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _same_device(*tensors) -> None:
    devs = {t.device for t in tensors if t is not None}
    if len(devs) > 1:
        raise ValueError(f"all tensors of one call must be on one device, got {sorted(map(str, devs))}")


def _ld(t: torch.Tensor) -> int:
    return t.stride(0) if t.dim() == 2 and t.shape[0] > 1 else t.shape[-1]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _workspace(ws, nbytes: int, device):
    """A caller's workspace must be a contiguous tensor on the call's device;
    without one, a zero-filled one of the required size is allocated."""
    if ws is not None:
        if not isinstance(ws, torch.Tensor):
            raise TypeError("workspace must be a torch.Tensor")
        if not ws.is_cuda or (device is not None and ws.device != torch.device(device)):
            raise ValueError(f"workspace must be on {device}, got {ws.device}")
        if not ws.is_contiguous():
            raise ValueError("workspace must be contiguous")
        return ws, ws.numel() * ws.element_size()
    if nbytes == 0:
        return None, 0
    return torch.zeros(nbytes, dtype=torch.uint8, device=device), nbytes


def _out(out, shape, like: torch.Tensor, name: str, contiguous: bool = True):
    """An output given by the caller must have the right shape, lie on the
    same device as `like` and, unless the C ABI takes its row stride
    (contiguous=False), be contiguous."""
    if out is None:
        return torch.empty(shape, dtype=torch.bfloat16, device=like.device)
    _check_tensor(out, name, len(shape), contiguous=contiguous, on_gpu=False)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(out.shape)}, expected {tuple(shape)}")
    if out.device != like.device:
        raise ValueError(f"{name} is on {out.device}, expected {like.device}")
    return out


class HipEvent:
    """A hipEvent_t created with hipEventDisableTiming (for stream fork/join)."""

    _hip = None

    def __init__(self):
        if HipEvent._hip is None:
            HipEvent._hip = ctypes.CDLL("libamdhip64.so")
        torch.cuda.init()
        h = ctypes.c_void_p()
        err = HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(0x2))
        if err != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({err})")
        self.handle = h

    def __del__(self):
        # type(self), not the module global: at interpreter exit the module's
        # globals may already be gone.
        hip = type(self)._hip
        if getattr(self, "handle", None) and hip is not None:
            hip.hipEventDestroy(self.handle)
            self.handle = None


# ---- entry points -----------------------------------------------------------

def skinny_gemm(A: torch.Tensor, W: torch.Tensor, residual: torch.Tensor | None = None, *,
                out: torch.Tensor | None = None, cfg: dict | None = None,
                workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """out = bf16(A @ W^T + residual).  A [M,K], W [N,K], residual [M,N]."""
    _check_tensor(A, "A", 2)
    _check_tensor(W, "W", 2)
    M, K = A.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError(f"A is [{M},{K}] but W is [{N},{K2}]")
    if residual is not None:
        _check_tensor(residual, "residual", 2)
        if tuple(residual.shape) != (M, N):
            raise ValueError("residual must be [M, N]")
    _same_device(A, W, residual)
    out = _out(out, (M, N), A, "out", contiguous=False)
    c = _config(cfg) if cfg is not None else None
    need = (sg_config_workspace_bytes(cfg, M, N) if cfg is not None
            else sg_workspace_bytes(SG_OP_GEMM, M, N, K))
    ws, ws_bytes = _workspace(workspace, need, A.device)
    st = _lib.load().skinny_gemm(
        _ptr(A), _ld(A), _ptr(W), _ld(W), _ptr(residual),
        _ld(residual) if residual is not None else N, _ptr(out), _ld(out), M, N, K,
        ctypes.byref(c) if c is not None else None, _ptr(ws), ws_bytes, _stream(stream, A.device))
    _lib.check(st, "skinny_gemm")
    return out


def kda_qkvg_proj(x: torch.Tensor, w_qkvg: torch.Tensor, *, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Packed Q/K/V/G projection: out = bf16(x @ w_qkvg^T), all contiguous."""
    _check_tensor(x, "x", 2)
    _check_tensor(w_qkvg, "w_qkvg", 2)
    M, K = x.shape
    N = w_qkvg.shape[0]
    if w_qkvg.shape[1] != K or not x.is_contiguous() or not w_qkvg.is_contiguous():
        raise ValueError("x [M,K] and w_qkvg [N,K] must be contiguous with matching K")
    _same_device(x, w_qkvg)
    out = _out(out, (M, N), x, "out")
    ws, ws_bytes = _workspace(workspace, sg_workspace_bytes(SG_OP_GEMM, M, N, K), x.device)
    st = _lib.load().kda_qkvg_proj(_ptr(x), _ptr(w_qkvg), _ptr(out), M, N, K, _ptr(ws), ws_bytes,
                                   _stream(stream, x.device))
    _lib.check(st, "kda_qkvg_proj")
    return out


def kda_fab_fb_proj_fused(*args, **kwargs):
    """kda_fab_fb_proj as one launch (the in-launch F_A/beta -> F_B hand-off):
    same arguments and results.  A workspace given by the caller must have
    been zero-filled once before its first use by this call."""
    return kda_fab_fb_proj(*args, _entry="kda_fab_fb_proj_fused", **kwargs)


def kda_fab_fb_proj(x: torch.Tensor, w_ab: torch.Tensor, w_b: torch.Tensor, rank: int = 128, *,
                    want_f_a: bool = False, f_a: torch.Tensor | None = None,
                    beta: torch.Tensor | None = None, g1: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, stream=None,
                    _entry: str = "kda_fab_fb_proj"):
    """F_A/beta -> F_B branch.  Returns (g1, beta) or (g1, beta, f_a) if want_f_a."""
    for t, n in ((x, "x"), (w_ab, "w_ab"), (w_b, "w_b")):
        _check_tensor(t, n, 2)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    M, K = x.shape
    n_ab = w_ab.shape[0]
    n_b = w_b.shape[0]
    if w_ab.shape[1] != K or w_b.shape[1] != rank:
        raise ValueError("w_ab must be [n_ab, K] and w_b [n_b, rank]")
    _same_device(x, w_ab, w_b)
    beta = _out(beta, (M, n_ab - rank), x, "beta")
    g1 = _out(g1, (M, n_b), x, "g1")
    if f_a is not None:
        f_a = _out(f_a, (M, rank), x, "f_a")
    elif want_f_a:
        f_a = torch.empty((M, rank), dtype=torch.bfloat16, device=x.device)
    ws, ws_bytes = _workspace(workspace, sg_workspace_bytes(SG_OP_FAB_FB, M, n_ab, K), x.device)
    st = getattr(_lib.load(), _entry)(_ptr(x), _ptr(w_ab), _ptr(w_b), _ptr(f_a), _ptr(beta),
                                      _ptr(g1), M, K, n_ab, rank, n_b, _ptr(ws), ws_bytes,
                                      _stream(stream, x.device))
    _lib.check(st, _entry)
    return (g1, beta, f_a) if f_a is not None else (g1, beta)


def kda_projection_overlap(x: torch.Tensor, packed_w: torch.Tensor, w_b: torch.Tensor, *,
                           n_qkvg: int = 4096, n_ab: int = 136, rank: int = 128,
                           qkvg: torch.Tensor | None = None, beta: torch.Tensor | None = None,
                           g1: torch.Tensor | None = None, ws_main: torch.Tensor | None = None,
                           ws_aux: torch.Tensor | None = None, main_stream=None, aux_stream=None,
                           fork: HipEvent | None = None, join: HipEvent | None = None):
    """QKVG on main_stream, F_A/beta -> F_B on aux_stream.  Returns (qkvg, g1, beta).

    With aux_stream, fork or join None the branches run one after the other on
    main_stream."""
    for t, n in ((x, "x"), (packed_w, "packed_w"), (w_b, "w_b")):
        _check_tensor(t, n, 2)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    M, K = x.shape
    n_b = w_b.shape[0]
    if packed_w.shape != (n_qkvg + n_ab, K) or w_b.shape[1] != rank:
        raise ValueError("packed_w must be [n_qkvg + n_ab, K] and w_b [n_b, rank]")
    _same_device(x, packed_w, w_b)
    qkvg = _out(qkvg, (M, n_qkvg), x, "qkvg")
    beta = _out(beta, (M, n_ab - rank), x, "beta")
    g1 = _out(g1, (M, n_b), x, "g1")
    wsm, wsm_bytes = _workspace(ws_main, sg_kda_workspace_bytes(0, M, K, n_qkvg, n_ab), x.device)
    wsa, wsa_bytes = _workspace(ws_aux, sg_kda_workspace_bytes(1, M, K, n_qkvg, n_ab), x.device)
    st = _lib.load().kda_projection_overlap(
        _ptr(x), _ptr(packed_w), _ptr(w_b), _ptr(qkvg), _ptr(beta), _ptr(g1), M, K, n_qkvg, n_ab,
        rank, n_b, _ptr(wsm), wsm_bytes, _ptr(wsa), wsa_bytes, _stream(main_stream, x.device),
        ctypes.c_void_p(aux_stream.cuda_stream) if aux_stream is not None else None,
        fork.handle if fork is not None else None, join.handle if join is not None else None)
    _lib.check(st, "kda_projection_overlap")
    return qkvg, g1, beta


def kda_projection_fused(x: torch.Tensor, packed_w: torch.Tensor, w_b: torch.Tensor, *,
                         n_qkvg: int = 4096, n_ab: int = 136, rank: int = 128,
                         qkvg: torch.Tensor | None = None, beta: torch.Tensor | None = None,
                         g1: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         stream=None):
    """The KDA projection as one launch (a helper wave per Q/K/V/G workgroup
    runs the F_A/beta -> F_B chain).  Returns (qkvg, g1, beta).  A workspace
    given by the caller must have been zero-filled once before its first use
    by this call and not altered since."""
    for t, n in ((x, "x"), (packed_w, "packed_w"), (w_b, "w_b")):
        _check_tensor(t, n, 2, contiguous=True)
    M, K = x.shape
    n_b = w_b.shape[0]
    if packed_w.shape != (n_qkvg + n_ab, K) or w_b.shape[1] != rank:
        raise ValueError("packed_w must be [n_qkvg + n_ab, K] and w_b [n_b, rank]")
    _same_device(x, packed_w, w_b)
    qkvg = _out(qkvg, (M, n_qkvg), x, "qkvg")
    beta = _out(beta, (M, n_ab - rank), x, "beta")
    g1 = _out(g1, (M, n_b), x, "g1")
    ws, ws_bytes = _workspace(workspace, sg_kda_workspace_bytes(SG_KDA_ONE_LAUNCH, M, K, n_qkvg, n_ab),
                              x.device)
    st = _lib.load().kda_projection_fused(
        _ptr(x), _ptr(packed_w), _ptr(w_b), _ptr(qkvg), _ptr(beta), _ptr(g1), M, K, n_qkvg, n_ab,
        rank, n_b, _ptr(ws), ws_bytes, _stream(stream, x.device))
    _lib.check(st, "kda_projection_fused")
    return qkvg, g1, beta


def kda_projection_noalloc(x: torch.Tensor, packed_w: torch.Tensor, w_b: torch.Tensor, *,
                           n_qkvg: int = 4096, n_ab: int = 136, rank: int = 128,
                           qkvg: torch.Tensor, beta: torch.Tensor, g1: torch.Tensor,
                           main_stream=None, aux_stream=None, fork: HipEvent | None = None,
                           join: HipEvent | None = None):
    """kda_projection_overlap with its workspaces in the library's own
    per-GPU device array: no allocation anywhere, so the outputs must be
    given.  Calls that may overlap on one GPU must not be issued."""
    for t, n in ((x, "x"), (packed_w, "packed_w"), (w_b, "w_b")):
        _check_tensor(t, n, 2, contiguous=True)
    M, K = x.shape
    n_b = w_b.shape[0]
    if packed_w.shape != (n_qkvg + n_ab, K) or w_b.shape[1] != rank:
        raise ValueError("packed_w must be [n_qkvg + n_ab, K] and w_b [n_b, rank]")
    _same_device(x, packed_w, w_b)
    if qkvg is None or beta is None or g1 is None:
        raise ValueError("kda_projection_noalloc allocates nothing: pass qkvg, beta and g1")
    qkvg = _out(qkvg, (M, n_qkvg), x, "qkvg")
    beta = _out(beta, (M, n_ab - rank), x, "beta")
    g1 = _out(g1, (M, n_b), x, "g1")
    st = _lib.load().kda_projection_noalloc(
        _ptr(x), _ptr(packed_w), _ptr(w_b), _ptr(qkvg), _ptr(beta), _ptr(g1), M, K, n_qkvg, n_ab,
        rank, n_b, _stream(main_stream, x.device),
        ctypes.c_void_p(aux_stream.cuda_stream) if aux_stream is not None else None,
        fork.handle if fork is not None else None, join.handle if join is not None else None)
    _lib.check(st, "kda_projection_noalloc")
    return qkvg, g1, beta


def latent_moe_tail_fused(*args, **kwargs):
    """latent_moe_tail with the GEMM's K-split sum inside its launch: same
    arguments and results.  A workspace given by the caller must have been
    zero-filled once before its first use by this call and not altered
    since."""
    return latent_moe_tail(*args, _entry="latent_moe_tail_fused", **kwargs)


def latent_moe_tail(latent: torch.Tensor, gamma: torch.Tensor, w_up: torch.Tensor,
                    shared: torch.Tensor | None = None, eps: float = 1e-6, *,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                    stream=None, _entry: str = "latent_moe_tail") -> torch.Tensor:
    """out = bf16(shared + RMSNorm(latent; gamma, eps) @ w_up^T)."""
    _check_tensor(latent, "latent", 2)
    _check_tensor(w_up, "w_up", 2)
    if not isinstance(gamma, torch.Tensor) or gamma.dim() != 1 or gamma.dtype not in _16BIT:
        raise ValueError("gamma must be a 1-D bf16 tensor")
    M, d = latent.shape
    D = w_up.shape[0]
    if w_up.shape[1] != d or gamma.shape[0] != d:
        raise ValueError("w_up must be [d_hidden, d_latent] and gamma [d_latent]")
    for t, n in ((latent, "latent"), (w_up, "w_up"), (gamma, "gamma")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if shared is not None:
        _check_tensor(shared, "shared", 2)
        if tuple(shared.shape) != (M, D) or not shared.is_contiguous():
            raise ValueError("shared must be a contiguous [M, d_hidden] tensor")
    _same_device(latent, gamma, w_up, shared)
    out = _out(out, (M, D), latent, "out")
    op = SG_OP_LATENT_TAIL_FUSED if _entry == "latent_moe_tail_fused" else SG_OP_LATENT_TAIL
    ws, ws_bytes = _workspace(workspace, sg_workspace_bytes(op, M, D, d), latent.device)
    st = getattr(_lib.load(), _entry)(_ptr(latent), _ptr(gamma), ctypes.c_float(eps), _ptr(w_up),
                                      _ptr(shared), _ptr(out), M, d, D, _ptr(ws), ws_bytes,
                                      _stream(stream, latent.device))
    _lib.check(st, _entry)
    return out
