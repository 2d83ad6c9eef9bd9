"""The environment the library reads once per process (no GPU needed):

* SKINNY_GEMM_LOG prints every configuration choice on stderr, with where it
  came from (rule, measured table, override, the KDA pairing);
* SKINNY_GEMM_TABLE installs override entries before the first choice; a
  malformed or unsupported value is reported and ignored, and a later
  sg_set_table_override replaces what it installed.

Each case runs in a fresh interpreter, since the environment is read once.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys
from pathlib import Path

import pytest

from bf16_skinny_gemm_02_amd import _lib

ROOT = Path(__file__).resolve().parent.parent
N, K = 4096, 7168
ENTRY = dict(N=N, K=K, m_lo=2, m_hi=4, kind=5, rows=32, waves=4, k_unroll=3, k_split=2)
ENTRY_TEXT = "4096,7168,2,4,5,32,4,3,2"

PROBE = r"""
import json, sys
import bf16_skinny_gemm_02_amd as sg
out = {"select": {M: sg.sg_select(M, %(N)d, %(K)d) for M in (1, 3, 5)}}
out["kda"] = sg.sg_kda_select(sg.SG_KDA_QKVG, 8, %(K)d, %(N)d, 136)
if "--clear" in sys.argv:
    sg.sg_set_table_override([])
    out["cleared"] = sg.sg_select(3, %(N)d, %(K)d)
print(json.dumps(out))
""" % dict(N=N, K=K)


def _run(env_extra: dict, *args: str):
    env = {k: v for k, v in os.environ.items() if not k.startswith("SKINNY_GEMM_")}
    env.update(env_extra)
    env["PYTHONPATH"] = str(ROOT) + os.pathsep + env.get("PYTHONPATH", "")
    p = subprocess.run([sys.executable, "-c", PROBE, *args], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stderr
    data = json.loads(p.stdout.strip().splitlines()[-1])
    data["select"] = {int(m): c for m, c in data["select"].items()}
    lines = [ln for ln in p.stderr.splitlines() if ln.startswith("skinny_gemm:")]
    return data, lines


@pytest.fixture(scope="module")
def default():
    if not _lib.LIB_PATH.exists():
        pytest.fail(f"{_lib.LIB_PATH} not built: run `python -m bf16_skinny_gemm_02_amd.build`")
    data, lines = _run({})
    assert lines == []  # nothing is printed unless asked for
    return data


def _full(entry: dict, M: int) -> dict:
    from bf16_skinny_gemm_02_amd import tune
    return tune._full(entry, M, entry["N"])


def test_log_prints_each_choice_and_its_source(default):
    data, lines = _run({"SKINNY_GEMM_LOG": "1"})
    assert data == default  # logging changes no choice
    sel = [ln for ln in lines if " select " in ln]
    assert len(sel) == 3
    for ln, M in zip(sel, (1, 3, 5)):
        c = default["select"][M]
        assert f"M={M} N={N} K={K} -> " in ln
        assert f"k_split={c['k_split']} grid={c['grid']}" in ln
        assert ln.endswith("(measured table)") or ln.endswith("(rule)")
    kda = [ln for ln in lines if "kda Q/K/V/G" in ln]
    assert len(kda) == 1 and "M=8" in kda[0] and "(one-round 128-row pairing)" in kda[0]
    assert _run({"SKINNY_GEMM_LOG": "0"})[1] == []


def test_table_from_the_environment_is_installed(default):
    data, lines = _run({"SKINNY_GEMM_TABLE": f" ;{ENTRY_TEXT}; ", "SKINNY_GEMM_LOG": "1"})
    assert data["select"][3] == _full(ENTRY, 3)
    assert data["select"][1] == default["select"][1]
    assert data["select"][5] == default["select"][5]
    assert any("installed 1 entries" in ln for ln in lines)
    assert any(" select M=3 " in ln and ln.endswith("(override)") for ln in lines)


def test_api_override_replaces_the_environment_table(default):
    data, _ = _run({"SKINNY_GEMM_TABLE": ENTRY_TEXT}, "--clear")
    assert data["select"][3] == _full(ENTRY, 3)
    assert data["cleared"] == default["select"][3]


@pytest.mark.parametrize("text,why", [
    ("4096,7168,2,4,5,32,4,3", "malformed"),            # eight fields
    ("4096,7168,2,4,5,32,4,3,2,1", "malformed"),        # ten fields
    ("4096;7168", "malformed"),
    ("4096,7168,2,4,5,32,4,3,x", "malformed"),
    ("4096,7168,2,17,5,32,4,3,2", "unsupported entry"),  # no wave-split instance at M = 17
    ("4096,7168,4,2,5,32,4,3,2", "invalid entry"),       # m_hi < m_lo
    (";".join([ENTRY_TEXT] * 65), "malformed"),          # more entries than the table holds
])
def test_bad_environment_table_is_reported_and_ignored(default, text, why):
    data, lines = _run({"SKINNY_GEMM_TABLE": text})
    assert data == default
    assert lines == [f"skinny_gemm: SKINNY_GEMM_TABLE ignored ({why})"]
