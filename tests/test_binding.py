"""Argument marshalling of the Python binding, on any host.

The binding hands raw pointers to the C ABI, which trusts the layout it is
told: an output the ABI writes as contiguous rows must be contiguous, a
caller-supplied f_a must have its full [M, rank] shape, and a workspace must
be device memory of the call's device.  These checks run before any pointer
is taken, so they are testable on CPU tensors (the device check comes after
the layout checks).
"""
from __future__ import annotations

import pytest
import torch

import bf16_skinny_gemm_02_amd as sg

CUDA0 = torch.device("cuda:0")


class _FakeCuda:
    """Stands in for a GPU tensor where only `.device` is read."""
    device = CUDA0


def test_strided_output_is_refused():
    base = torch.zeros((4, 16), dtype=torch.bfloat16)
    beta = base[:, ::2]                      # last-dim stride 2
    with pytest.raises(ValueError, match="unit stride"):
        sg._out(beta, (4, 8), _FakeCuda(), "beta")
    rows = base[:, :8]                       # unit stride, row stride 16: not contiguous
    with pytest.raises(ValueError, match="contiguous"):
        sg._out(rows, (4, 8), _FakeCuda(), "beta")


def test_strided_output_allowed_where_the_abi_takes_a_stride():
    rows = torch.zeros((4, 16), dtype=torch.bfloat16)[:, :8]
    # skinny_gemm passes ldc: only the device differs here.
    with pytest.raises(ValueError, match="is on cpu"):
        sg._out(rows, (4, 8), _FakeCuda(), "out", contiguous=False)


def test_undersized_f_a_is_refused():
    f_a = torch.zeros((2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"shape \(2, 64\), expected \(2, 128\)"):
        sg._out(f_a, (2, 128), _FakeCuda(), "f_a")


def test_output_dtype_and_rank_are_checked():
    with pytest.raises(TypeError):
        sg._out(torch.zeros((2, 8), dtype=torch.float32), (2, 8), _FakeCuda(), "g1")
    with pytest.raises(ValueError, match="2-D"):
        sg._out(torch.zeros((16,), dtype=torch.bfloat16), (2, 8), _FakeCuda(), "g1")


def test_cpu_workspace_is_refused():
    ws = torch.zeros(4096, dtype=torch.uint8)
    with pytest.raises(ValueError, match="workspace must be on cuda:0"):
        sg._workspace(ws, 1024, CUDA0)


def test_workspace_type_is_checked():
    with pytest.raises(TypeError):
        sg._workspace(bytearray(16), 16, CUDA0)


def test_no_workspace_needed_passes_null():
    assert sg._workspace(None, 0, CUDA0) == (None, 0)


def test_mixed_devices_are_refused():
    a = torch.zeros(1)

    class Other:
        device = CUDA0

    with pytest.raises(ValueError, match="one device"):
        sg._same_device(a, Other())
    sg._same_device(a, None, torch.zeros(2))
