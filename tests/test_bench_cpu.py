"""Host logic of bench.py's live byte-counter measurement: the grouping of a
rocprofv3 results database's counter records, the copy calibration, the
launch-weighted mean, and the refusal paths (no profiler, nested profiling)."""
import importlib.util
import os
import sqlite3

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


CFG = {"n_cand": 96, "tokens": 4096, "dim": 3072, "hidden": 12288, "blocks": 4, "steps": 6}


def test_variants_cover_every_gemm_launch_of_a_step(bench):
    v = bench.gemm_variants(CFG)
    assert {k: n for k, (_, n) in v.items()} == {"gelu_mxfp4": 24, "residual": 18, "euler": 5, "euler_reward": 1}
    # two linears per block and Euler step
    assert sum(n for _, n in v.values()) == 2 * CFG["blocks"] * CFG["steps"]
    assert len({t for t, _ in v.values()}) == 4


def _db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?)", rows)
    con.commit()
    con.close()


def _name(tmpl):
    return f"void fp4r::(anonymous namespace)::{tmpl}(unsigned char const*, int)"


def test_counter_records_are_grouped_by_kernel(bench, tmp_path):
    v = bench.gemm_variants(CFG)
    rows = [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 262144.0), ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 262144.0),
            ("__amd_rocclr_copyBuffer", "WRITE_SIZE", 999.0),           # another counter: ignored
            ("void quant_mx_rmsnorm_wave_kernel<0, 6, true>(float const*)", "FETCH_SIZE", 5.0)]
    for i, (tmpl, _) in enumerate(v.values()):
        rows += [(_name(tmpl), "FETCH_SIZE", 1000.0 * (i + 1)), (_name(tmpl), "FETCH_SIZE", 1000.0 * (i + 1) + 2)]
    # a kernel whose template arguments extend another's must not be taken for it
    rows.append((_name("gemm_fp4_kernel<0, 3, 2, 1>"), "FETCH_SIZE", 7.0))
    db = str(tmp_path / "f.db")
    _db(db, rows)
    kib = bench.counter_kib(db, "FETCH_SIZE", v)
    assert kib["copy"] == [262144.0, 262144.0]
    for i, name in enumerate(v):
        assert kib[name] == [1000.0 * (i + 1), 1000.0 * (i + 1) + 2]


def test_a_missing_variant_fails_the_pass(bench, tmp_path):
    v = bench.gemm_variants(CFG)
    rows = [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 1.0)]
    rows += [(_name(t), "FETCH_SIZE", 1.0) for name, (t, _) in v.items() if name != "euler"]
    db = str(tmp_path / "g.db")
    _db(db, rows)
    assert bench.counter_kib(db, "FETCH_SIZE", v) is None


def test_weighted_mean_per_launch(bench):
    v = bench.gemm_variants(CFG)
    per = {"gelu_mxfp4": {"read_GB": 11.0, "write_GB": 2.0}, "residual": {"read_GB": 18.0, "write_GB": 5.0},
           "euler": {"read_GB": 24.0, "write_GB": 5.0}, "euler_reward": {"read_GB": 25.0, "write_GB": 5.0}}
    want = (24 * 13.0 + 18 * 23.0 + 5 * 29.0 + 1 * 30.0) / 48 * 1e9
    assert bench.weighted_traffic(per, v) == pytest.approx(want, rel=1e-12)


def test_no_profiler_on_path_is_reported_not_raised(bench, monkeypatch, tmp_path):
    monkeypatch.setenv("PATH", str(tmp_path))
    res, why = bench.measure_traffic(CFG)
    assert res is None and "rocprofv3" in why


def test_nested_profiling_is_detected(bench):
    assert not bench._under_profiler({"PATH": "/usr/bin", "LD_PRELOAD": "/usr/lib/libother.so"})
    assert bench._under_profiler({"ROCPROFILER_LIBRARY_CTOR": "1"})
    assert bench._under_profiler({"LD_PRELOAD": "/opt/rocm/lib/librocprofiler-sdk-tool.so"})


def test_profile_fallback_is_the_recorded_figure_or_none(bench):
    # reported only while the GEMM sources hash to the recorded values
    assert bench.gemm_traffic() in (None, bench.GEMM_TRAFFIC["bytes_per_launch"])
