"""Build libskinny_gemm.so in-tree with hipcc for gfx950.

    python -m bf16_skinny_gemm_02_amd.build

Objects go to ``_build/`` at the repository root; the shared library is written
next to this file.  Every HIP source is compiled with packed-FP32 instructions
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = ROOT / "_build"
LIB = PKG / "libskinny_gemm.so"
ARCH = "gfx950"

SOURCES = ["gemv.hip", "smallk.hip", "mfma.hip", "noalloc.hip", "abi.cpp", "dispatch.cpp"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libskinny_gemm")


def _common_flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: Path, obj: Path) -> None:
    cmd = [_hipcc(), *_common_flags(), "-x", "hip", "-c", str(src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src.name} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


def build(jobs: int | None = None, verbose: bool = True) -> Path:
    BUILD.mkdir(exist_ok=True)
    objs = []
    jobs = jobs or min(8, len(SOURCES))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = []
        for name in SOURCES:
            obj = BUILD / (name + ".o")
            objs.append(obj)
            futs.append(ex.submit(_compile, CSRC / name, obj))
        for f in futs:
            f.result()
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *map(str, objs), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
