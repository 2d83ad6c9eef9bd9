"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The configuration table (csrc/dispatch.cpp) and the C oracle (oracle/oracle.c)
are plain host C/C++.  Each is built here with
``-fsanitize=address,undefined -fno-sanitize-recover=all`` together with a
small driver (tests/sanitize/), run over a grid of inputs, and its output
compared with the normal build: the selection mirror for the table, the
OpenMP build of the oracle for the oracle.  Any out-of-bounds access,
overflow or other undefined behaviour aborts the driver and fails the test.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

import numpy as np
import pytest

import oracle
import synth
from oracle import selection

ROOT = Path(__file__).resolve().parent.parent
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-O1", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


@pytest.fixture(scope="module")
def select_driver(tmp_path_factory):
    _need("g++")
    out = tmp_path_factory.mktemp("san") / "select_driver"
    subprocess.run(["g++", "-std=c++17", *SAN, f"-I{ROOT / 'include'}",
                    str(ROOT / "tests" / "sanitize" / "select_driver.cpp"),
                    str(ROOT / "bf16_skinny_gemm_02_amd" / "csrc" / "dispatch.cpp"),
                    "-o", str(out)], check=True)
    return out


@pytest.fixture(scope="module")
def oracle_driver(tmp_path_factory):
    _need("gcc")
    out = tmp_path_factory.mktemp("san") / "oracle_driver"
    subprocess.run(["gcc", "-std=c11", *SAN, str(ROOT / "tests" / "sanitize" / "oracle_driver.c"),
                    str(ROOT / "oracle" / "oracle.c"), "-lm", "-o", str(out)], check=True)
    return out


def _fields(cfg):
    return [cfg[f] for f in selection.FIELDS]


def test_config_table_under_sanitizers(select_driver):
    res = subprocess.run([str(select_driver)], capture_output=True, text=True, env=ENV, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    n = 0
    for line in res.stdout.splitlines():
        head, _, tail = line.partition(" : ")
        parts = head.split()
        vals = tail.split()
        fn, args = parts[0], [int(v) for v in parts[1:]]
        if fn == "select":
            st, cfg = selection.select(*args[:3], bool(args[3]))
            assert int(vals[0]) == st, line
            if st == selection.OK:
                assert [int(v) for v in vals[1:]] == _fields(cfg), line
        elif fn == "ws":
            op, M, N, K = args
            if op == 0 and M >= 0:
                st, cfg = selection.select(M, N, K)
                want = 0
                if st == selection.OK and cfg["kind"] != selection.NONE and cfg["k_split"] > 1:
                    want = (cfg["k_split"] * M * N * 4 + 255) // 256 * 256
                assert int(vals[0]) == want, line
        elif fn == "kda":
            st, cfg = selection.kda_select(*args)
            assert int(vals[0]) == st, line
            if st == selection.OK:
                assert [int(v) for v in vals[1:]] == _fields(cfg), line
        elif fn == "kdaws":
            which, M, K, nq, nab = args
            if which in (0, 1):
                assert int(vals[0]) == selection.kda_workspace_bytes(which, M, K, nq, nab), line
        elif fn == "gate":
            assert int(vals[0]) == int(selection.overlap_gate(*args)), line
        elif fn == "null":
            assert int(vals[0]) == selection.INVALID_ARG
        n += 1
    assert n > 20000


def _run_oracle(driver, text):
    res = subprocess.run([str(driver)], input=text, capture_output=True, text=True, env=ENV,
                         timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    return np.array([int(v) for v in res.stdout.split()], dtype=np.uint16)


def _nums(a):
    return " ".join(str(int(v)) for v in np.asarray(a, dtype=np.uint16).ravel())


@pytest.mark.parametrize("M,N,K,res", [(1, 7, 40, False), (3, 5, 264, True), (4, 9, 1000, True),
                                       (2, 3, 0, True), (5, 1, 8, False)])
def test_oracle_gemm_under_sanitizers(oracle_driver, M, N, K, res):
    A, W, R = synth.gemm_inputs(M, N, K, seed=17 + M + N + K, residual=res)
    text = f"gemm {M} {N} {K} {int(res)}\n{_nums(A)}\n{_nums(W)}\n" + (f"{_nums(R)}\n" if res else "")
    got = _run_oracle(oracle_driver, text)
    _, want = oracle.gemm(A, W, R)
    assert np.array_equal(got, want.ravel())


@pytest.mark.parametrize("M,d,D,shared", [(1, 64, 5, True), (3, 264, 7, False), (2, 2048, 3, True)])
def test_oracle_tail_under_sanitizers(oracle_driver, M, d, D, shared):
    L, gamma, w_up, S = synth.tail_inputs(M, seed=23 + M, d=d, D=D)
    text = (f"tail {M} {d} {D} {int(shared)} 1\n{_nums(L)}\n{_nums(gamma)}\n{_nums(w_up)}\n" +
            (f"{_nums(S)}\n" if shared else ""))
    got = _run_oracle(oracle_driver, text)
    for variant in (0, 1):
        _, want = oracle.latent_tail(L, gamma, 1e-6, w_up, S if shared else None, variant=variant)
        part = got[variant * M * D:(variant + 1) * M * D]
        assert np.array_equal(part, want.ravel()), variant


def test_oracle_rounding_under_sanitizers(oracle_driver):
    vals = [0.0, -0.0, 1.0, 1.00390625, 1.005859375, -3.5e38, 3.4e38, 1e-40, -1e-45,
            float("inf"), float("-inf"), float("nan"), 2.0 ** -133, 2.0 ** -134, 123.456]
    text = f"round {len(vals)}\n" + " ".join(float(v).hex() for v in vals) + "\n"
    got = _run_oracle(oracle_driver, text)
    want = oracle.round_bf16(np.array(vals, dtype=np.float64))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("text,installed", [
    ("4096,7168,2,4,5,32,4,3,2", True),
    (" ; 4096 , 7168 , 2 , 4 , 5 , 32 , 4 , 3 , 2 ;;", True),
    ("4096,7168,2,4,5,32,4,3", False),
    ("99999999999999999999,7168,2,4,5,32,4,3,2", False),
    ("-4096,7168,2,4,5,32,4,3,2", False),
    (",,,,,,,,", False),
    ("4096,7168,2,4,5,32,4,3,2;" * 70, False),
    ("x" * 5000, False),
])
def test_environment_table_parser_under_sanitizers(select_driver, text, installed):
    # The environment is read by the first configuration call; whatever the
    # text, it is installed or reported, and nothing reads out of bounds.
    env = dict(ENV, SKINNY_GEMM_TABLE=text, SKINNY_GEMM_LOG="1")
    res = subprocess.run([str(select_driver)], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    head = [ln for ln in res.stderr.splitlines() if "SKINNY_GEMM_TABLE" in ln]
    assert len(head) == 1
    assert ("installed 1 entries" in head[0]) == installed, head
