"""ctypes loader for libskinny_gemm.so (the C ABI in include/skinny_gemm.h).

The library is built in-tree by ``bf16_skinny_gemm_02_amd.build``.  There is no
fallback: if the shared library is missing or fails to load, every entry point
raises.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libskinny_gemm.so"

SG_OK = 0
SG_ERR_INVALID_ARG = -1
SG_ERR_UNSUPPORTED = -2
SG_ERR_MISALIGNED = -3
SG_ERR_WORKSPACE = -4
SG_ERR_HIP = -5

SG_KIND_NONE = 0
SG_KIND_GEMV_ROW = 1
SG_KIND_GEMV_SPLITK = 2
SG_KIND_GEMV_SMALLK = 3
SG_KIND_MFMA_TILE = 4
SG_KIND_MFMA_WAVESPLIT = 5
SG_KIND_MFMA_BLOCK = 6

SG_OP_GEMM = 0
SG_OP_FAB_FB = 1
SG_OP_LATENT_TAIL = 2
SG_OP_LATENT_TAIL_FUSED = 3

SG_KDA_QKVG = 0
SG_KDA_FAB = 1
SG_KDA_FAB_ALONE = 2
SG_KDA_ONE_LAUNCH = 3

# Every extern "C" symbol declared in include/skinny_gemm.h.
EXPORTED_SYMBOLS = (
    "sg_select", "sg_overlap_gate", "sg_overlap_max_tokens", "sg_workspace_bytes",
    "sg_kda_select", "sg_kda_workspace_bytes",
    "sg_strerror", "sg_version", "skinny_gemm", "kda_qkvg_proj", "kda_fab_fb_proj",
    "kda_projection_overlap", "latent_moe_tail", "kda_projection_noalloc", "kda_fab_fb_proj_fused",
    "kda_projection_fused", "sg_kda_one_launch_fits", "latent_moe_tail_fused",
    "sg_config_supported", "sg_config_workspace_bytes", "sg_tuned_table", "sg_set_table_override",
)


class SgConfig(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in
                ("kind", "m_tile", "rows", "waves", "k_split", "k_unroll", "grid", "nt_weights")]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


TABLE_FIELDS = ("N", "K", "m_lo", "m_hi", "kind", "rows", "waves", "k_unroll", "k_split")


class SgTableEntry(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in TABLE_FIELDS]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

_PROTOS = {
    "sg_select": (_i32, [_i32, _i32, _i32, _i32, ctypes.POINTER(SgConfig)]),
    "sg_overlap_gate": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "sg_overlap_max_tokens": (_i32, []),
    "sg_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "sg_kda_select": (_i32, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(SgConfig)]),
    "sg_kda_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "sg_strerror": (ctypes.c_char_p, [_i32]),
    "sg_version": (ctypes.c_char_p, []),
    "skinny_gemm": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i32, _i32, _i32,
                           ctypes.POINTER(SgConfig), _vp, _sz, _vp]),
    "kda_qkvg_proj": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "kda_fab_fb_proj": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                               _vp, _sz, _vp]),
    "kda_projection_overlap": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _vp, _sz, _vp, _sz, _vp, _vp, _vp, _vp]),
    "latent_moe_tail": (_i32, [_vp, _vp, ctypes.c_float, _vp, _vp, _vp, _i32, _i32, _i32,
                               _vp, _sz, _vp]),
    "kda_projection_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _vp, _vp, _vp, _vp]),
    "kda_fab_fb_proj_fused": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                     _vp, _sz, _vp]),
    "kda_projection_fused": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _vp, _sz, _vp]),
    "sg_kda_one_launch_fits": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "latent_moe_tail_fused": (_i32, [_vp, _vp, ctypes.c_float, _vp, _vp, _vp, _i32, _i32, _i32,
                                     _vp, _sz, _vp]),
    "sg_config_supported": (_i32, [ctypes.POINTER(SgConfig), _i32, _i32, _i32]),
    "sg_config_workspace_bytes": (_sz, [ctypes.POINTER(SgConfig), _i32, _i32]),
    "sg_tuned_table": (_i32, [ctypes.POINTER(ctypes.POINTER(SgTableEntry))]),
    "sg_set_table_override": (_i32, [ctypes.POINTER(SgTableEntry), _i32]),
}

# Hand-off header at the start of the one-launch workspaces (SG_FAB_HEADER_BYTES).
SG_FAB_HEADER_BYTES = 18432

# Per-GPU scratch of kda_projection_noalloc (SG_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 16 << 20

_lib = None


def load() -> ctypes.CDLL:
    """Load libskinny_gemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m bf16_skinny_gemm_02_amd.build` "
                "(the library has no CPU fallback)")
        lib = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in _PROTOS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class SkinnyGemmError(RuntimeError):
    pass


def check(status: int, what: str) -> None:
    if status == SG_OK:
        return
    msg = f"{what}: {load().sg_strerror(status).decode()} (status {status})"
    if status == SG_ERR_HIP:
        raise SkinnyGemmError(msg)
    raise ValueError(msg)
