"""The measured configuration table (no GPU).

The analogue of the pages' check that the configurations in use equal the
measured table ("Overlap low-M TP8 KDA projections",
test_kda_overlap_configs_match_measured_table):

* the table compiled into libskinny_gemm.so (sg_tuned_table, from
  csrc/tuned_table.inc) is exactly the measured table's chosen entries
  (bf16_skinny_gemm_02_amd/tuned_table.json), and the .inc and
  docs/config_table.md are what the tuner renders from that JSON;
* every chosen entry is the measured winner under the tuner's policy, and
  sg_select returns it at every M of its range; the compiled overlap gate is
  the one derived from the JSON's timings of both schedules;
* the support predicate, the per-configuration workspace and the override
  table that the tuner drives behave as the header states.
"""
from __future__ import annotations

import ctypes
import json
from pathlib import Path

import pytest

import bf16_skinny_gemm_02_amd as sg
from bf16_skinny_gemm_02_amd import _lib, tune
from bf16_skinny_gemm_02_amd.tune_gate import derive_gate
from oracle import selection

ROOT = Path(__file__).resolve().parent.parent


@pytest.fixture(scope="module")
def lib():
    if not _lib.LIB_PATH.exists():
        pytest.fail(f"{_lib.LIB_PATH} not built: run `python -m bf16_skinny_gemm_02_amd.build`")
    return _lib.load()


def _table():
    return json.loads(tune.JSON_PATH.read_text()) if tune.JSON_PATH.exists() else None


def test_compiled_table_is_the_measured_table(lib):
    table = _table()
    compiled = sg.sg_tuned_table()
    if table is None:
        assert compiled == []
        assert "{0, 0, 0, 0, 0, 0, 0, 0, 0}" in tune.INC_PATH.read_text()
        return
    assert compiled == tune.table_entries(table)
    assert tune.INC_PATH.read_text() == tune.render_inc(table)
    assert tune.MD_PATH.read_text() == tune.render_md(table)
    assert sg.sg_overlap_max_tokens() == table["overlap"]["max_tokens"]
    assert table["overlap"]["max_tokens"] == derive_gate(table["overlap"]["per_m"])


def test_chosen_entries_are_the_measured_winners():
    table = _table()
    if table is None:
        pytest.skip("no measured table yet")
    for b in table["buckets"]:
        assert b["chosen"] == tune.choose(b["candidates"], b["incumbent"], table["margin"]), b
        measured = [c for c in b["candidates"] if c["cfg"] == b["chosen"]]
        assert measured and measured[0]["total_us"] is not None, b
        assert len(measured[0]["us"]) == len(b["measured_at"])
        assert b["measured_at"] == sorted({b["m_lo"], b["m_hi"]})


def test_select_follows_the_table_at_every_m(lib):
    for e in sg.sg_tuned_table():
        for M in range(e["m_lo"], e["m_hi"] + 1):
            got = sg.sg_select(M, e["N"], e["K"])
            assert {f: got[f] for f in tune.FIELDS} == {f: e[f] for f in tune.FIELDS}, (e, M)
            assert got == tune._full(e, M, e["N"])
            assert sg.sg_config_supported(got, M, e["N"], e["K"])


def test_the_rule_only_yields_supported_configurations(lib):
    for N, K in ((4096, 7168), (136, 7168), (1024, 128), (7168, 2048), (4232, 7168), (300, 264),
                 (5200, 1000), (9000, 512), (8190, 264), (40, 8), (1, 7168), (100, 65536)):
        for M in list(range(1, 67)) + [100, 128, 129, 200, 256]:
            st, cfg = selection.select(M, N, K)
            assert st == selection.OK
            assert sg.sg_config_supported(cfg, M, N, K), (M, N, K, cfg)


def test_support_predicate_rejects_what_no_kernel_runs(lib):
    base = dict(kind=5, m_tile=8, rows=16, waves=4, k_split=1, k_unroll=3, grid=256, nt_weights=1)
    assert sg.sg_config_supported(base, 8, 4096, 7168)
    for bad in (dict(rows=36, grid=114), dict(rows=18, grid=228), dict(k_unroll=4),
                dict(m_tile=16), dict(grid=255), dict(waves=8), dict(k_split=0),
                dict(k_split=300, grid=256 * 300), dict(nt_weights=0)):
        assert not sg.sg_config_supported({**base, **bad}, 8, 4096, 7168), bad
    assert not sg.sg_config_supported(base, 17, 4096, 7168)  # wave-split tiles stop at 16 rows of M
    assert not sg.sg_config_supported({**base, "k_unroll": 2}, 8, 4096, 7168)  # 2 slots: M > 8
    assert sg.sg_config_supported({**base, "k_unroll": 2, "m_tile": 12}, 9, 4096, 7168)
    gemv = dict(kind=1, m_tile=1, rows=7, waves=4, k_split=1, k_unroll=16, grid=256, nt_weights=1)
    assert sg.sg_config_supported(gemv, 1, 7168, 2048)
    assert not sg.sg_config_supported(gemv, 1, 7168, 4096)        # 8 steps > 4 for 7 rows
    assert not sg.sg_config_supported({**gemv, "m_tile": 2}, 2, 7168, 2048)  # GEMV only at M = 1
    with pytest.raises(ValueError):
        sg.sg_config_supported(base, -1, 4096, 7168)


def test_every_candidate_the_tuner_can_time_is_a_supported_configuration(lib):
    for N, K, _ in tune.SHAPES.values():
        for lo, hi in tune.BUCKETS:
            n_ok = 0
            for c in tune.candidates(N, K, lo, hi):
                ok = [sg.sg_config_supported(tune._full(c, M, N), M, N, K) for M in (lo, hi)]
                n_ok += all(ok)
            assert n_ok >= (0 if (K <= 256 and hi <= 16) else 1), (N, K, lo, hi)


def test_config_workspace_bytes(lib):
    c = dict(kind=4, m_tile=32, rows=64, waves=4, k_split=3, k_unroll=3, grid=192, nt_weights=1)
    assert sg.sg_config_workspace_bytes(c, 20, 4096) == (3 * 20 * 4096 * 4 + 255) // 256 * 256
    assert sg.sg_config_workspace_bytes({**c, "k_split": 1}, 20, 4096) == 0
    assert lib.sg_config_workspace_bytes(None, 20, 4096) == 0


def test_override_replaces_the_table_and_is_validated(lib):
    N, K = 4096, 7168
    before = {M: sg.sg_select(M, N, K) for M in (1, 2, 4, 5)}
    entry = dict(N=N, K=K, m_lo=2, m_hi=4, kind=5, rows=32, waves=4, k_unroll=3, k_split=2)
    try:
        sg.sg_set_table_override([entry])
        for M in (2, 3, 4):
            got = sg.sg_select(M, N, K)
            assert got == tune._full(entry, M, N)
            assert sg.sg_workspace_bytes(sg.SG_OP_GEMM, M, N, K) == \
                (2 * M * N * 4 + 255) // 256 * 256
        assert sg.sg_select(1, N, K) == before[1] and sg.sg_select(5, N, K) == before[5]
        # an entry no kernel can run at some M of its range leaves the override unchanged
        with pytest.raises(ValueError):
            sg.sg_set_table_override([dict(entry, m_hi=17)])
        assert sg.sg_select(3, N, K) == tune._full(entry, 3, N)
        with pytest.raises(ValueError):
            sg.sg_set_table_override([entry] * 65)
        assert lib.sg_set_table_override(None, 1) == _lib.SG_ERR_INVALID_ARG
    finally:
        sg.sg_set_table_override([])
    assert {M: sg.sg_select(M, N, K) for M in (1, 2, 4, 5)} == before


def test_choose_keeps_the_incumbent_within_the_margin():
    inc = dict(kind=5, rows=16, waves=4, k_unroll=3, k_split=1)
    other = dict(inc, k_split=2)
    cands = [{"cfg": inc, "total_us": 10.1}, {"cfg": other, "total_us": 10.0},
             {"cfg": dict(inc, rows=32), "total_us": None}]
    assert tune.choose(cands, inc) == inc
    cands[1]["total_us"] = 9.5
    assert tune.choose(cands, inc) == other
    assert tune.choose([{"cfg": other, "total_us": None}], inc) == inc


def test_render_inc_of_an_empty_table_is_the_sentinel():
    text = tune.render_inc({"buckets": [], "overlap": {"max_tokens": 0, "per_m": []}})
    assert "{0, 0, 0, 0, 0, 0, 0, 0, 0}," in text
    assert "kTunedOverlapMaxTokens = 0;" in text
