"""Host logic of bench.py's live counter measurement: the grouping of a
rocprofv3 results database's counter records by dispatch, the
launch-weighted mean of the byte counts, the clock and MFMA-busy arithmetic,
and the refusal paths (no profiler, nested profiling)."""
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
    assert bench.gemm_variants(CFG)["gelu_mxfp4"][0] == "gemm_fp4_kernel<0, 5, 2>"       # fp32 hidden (default)
    assert bench.gemm_variants(dict(CFG, hidden_act="bf16"))["gelu_mxfp4"][0] == "gemm_fp4_kernel<0, 3, 2>"
    v = bench.gemm_variants(CFG)
    assert {k: n for k, (_, n) in v.items()} == {"gelu_mxfp4": 24, "residual": 18, "euler": 5, "euler_reward": 1}
    # two linears per block and Euler step
    assert sum(n for _, n in v.values()) == 2 * CFG["blocks"] * CFG["steps"]
    assert len({t for t, _ in v.values()}) == 4


def _db(path, rows):
    """rows: (dispatch_id, kernel_name, counter_name, value, start, end)"""
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (dispatch_id integer, kernel_name text, counter_name text, "
                "value real, start integer, end integer)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def _name(tmpl):
    return f"void fp4r::(anonymous namespace)::{tmpl}(unsigned char const*, int)"


def test_counter_records_are_grouped_by_kernel(bench, tmp_path):
    v = bench.gemm_variants(CFG)
    rows = [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 262144.0, 0, 10),
            (2, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 262144.0, 10, 20),
            (2, "__amd_rocclr_copyBuffer", "SQ_WAVES", 999.0, 10, 20),            # another counter: ignored
            (3, "void quant_mx_rmsnorm_wave_kernel<0, 6, true>(float const*)", "FETCH_SIZE", 5.0, 20, 30)]
    did = 10
    for i, (tmpl, _) in enumerate(v.values()):
        for j in range(2):
            rows.append((did, _name(tmpl), "FETCH_SIZE", 1000.0 * (i + 1) + 2 * j, 100 * did, 100 * did + 7 + j))
            did += 1
    # a kernel whose template arguments extend another's must not be taken for it
    rows.append((99, _name("gemm_fp4_kernel<0, 3, 2, 1>"), "FETCH_SIZE", 7.0, 0, 1))
    # a copy after the rollout's GEMMs (input generation) is not the calibration copy
    rows.append((500, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 123.0, 0, 1))
    db = str(tmp_path / "f.db")
    _db(db, rows)
    g = bench.counter_dispatches(db, ("FETCH_SIZE",), v)
    assert g["copy"] == [(10, {"FETCH_SIZE": 262144.0}), (10, {"FETCH_SIZE": 262144.0})]
    for i, name in enumerate(v):
        assert g[name] == [(7, {"FETCH_SIZE": 1000.0 * (i + 1)}), (8, {"FETCH_SIZE": 1000.0 * (i + 1) + 2})]


def test_two_counters_of_one_dispatch_are_joined(bench, tmp_path):
    v = bench.gemm_variants(CFG)
    c = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
    rows = [(1, "__amd_rocclr_copyBuffer", c[0], 1.0, 0, 5), (1, "__amd_rocclr_copyBuffer", c[1], 2.0, 0, 5)]
    did = 2
    for tmpl, _ in v.values():
        rows += [(did, _name(tmpl), c[0], 3.0 * did, 0, 9), (did, _name(tmpl), c[1], 5.0 * did, 0, 9)]
        did += 1
    rows.append((50, _name("gemm_fp4_kernel<0, 1, 2>"), c[0], 1.0, 0, 9))   # one counter missing: dropped
    db = str(tmp_path / "c.db")
    _db(db, rows)
    g = bench.counter_dispatches(db, c, v)
    for k, name in enumerate(v):
        d = k + 2
        assert g[name] == [(9, {c[0]: 3.0 * d, c[1]: 5.0 * d})]


def test_a_missing_variant_fails_the_pass(bench, tmp_path):
    v = bench.gemm_variants(CFG)
    rows = [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 1.0, 0, 1)]
    rows += [(i + 2, _name(t), "FETCH_SIZE", 1.0, 0, 1) for i, (name, (t, _)) in enumerate(v.items())
             if name != "euler"]
    db = str(tmp_path / "g.db")
    _db(db, rows)
    assert bench.counter_dispatches(db, ("FETCH_SIZE",), v) is None


def test_clock_and_mfma_busy(bench):
    # 8 XCDs of 2e9 active cycles each over 1 s: 2 GHz; MFMA busy on half the
    # 1024 SIMDs' cycles: 0.5. A second dispatch at 1 GHz and busy 0.25 weighs by
    # its cycles and time.
    d1 = (1e9, {"GRBM_GUI_ACTIVE": 8 * 2e9, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 2e9 * 1024})
    assert bench.clock_stats([d1]) == pytest.approx((2.0, 0.5))
    d2 = (1e9, {"GRBM_GUI_ACTIVE": 8 * 1e9, "SQ_VALU_MFMA_BUSY_CYCLES": 0.25 * 1e9 * 1024})
    clk, busy = bench.clock_stats([d1, d2])
    assert clk == pytest.approx(1.5) and busy == pytest.approx((0.5 * 2 + 0.25 * 1) / 3)


def test_weighted_mean_per_launch(bench):
    v = bench.gemm_variants(CFG)
    per = {"gelu_mxfp4": {"read_GB": 11.0, "write_GB": 2.0}, "residual": {"read_GB": 18.0, "write_GB": 5.0},
           "euler": {"read_GB": 24.0, "write_GB": 5.0}, "euler_reward": {"read_GB": 25.0, "write_GB": 5.0}}
    want = (24 * 13.0 + 18 * 23.0 + 5 * 29.0 + 1 * 30.0) / 48 * 1e9
    assert bench.weighted_traffic(per, v) == pytest.approx(want, rel=1e-12)


def test_no_profiler_on_path_is_reported_not_raised(bench, monkeypatch, tmp_path):
    monkeypatch.setenv("PATH", str(tmp_path))
    res, why = bench.measure_counters(CFG)
    assert res is None and "rocprofv3" in why


def test_nested_profiling_is_detected(bench):
    assert not bench._under_profiler({"PATH": "/usr/bin", "LD_PRELOAD": "/usr/lib/libother.so"})
    assert bench._under_profiler({"ROCPROFILER_LIBRARY_CTOR": "1"})
    assert bench._under_profiler({"LD_PRELOAD": "/opt/rocm/lib/librocprofiler-sdk-tool.so"})


def test_profile_fallback_is_the_recorded_figure_or_none(bench):
    # reported only while the GEMM sources hash to the recorded values, and for
    # the hidden activation the profile was taken with
    h = bench.GEMM_TRAFFIC["hidden"]
    assert bench.gemm_traffic(h) in (None, bench.GEMM_TRAFFIC["bytes_per_launch"])
    assert bench.gemm_traffic("f32" if h == "bf16" else "bf16") is None


def test_class_dispatches_are_kept_in_launch_order(bench, tmp_path):
    v = bench.gemm_variants(CFG)
    shapes = bench.class_shapes()
    assert len(shapes) == 6 and len({k for k, *_ in shapes}) == 6
    rows = [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 1.0, 0, 1)]
    rows += [(i + 2, _name(t), "FETCH_SIZE", 1.0, 0, 1) for i, (t, _) in enumerate(v.values())]
    n_cls = bench.PROBE_CLASS_LAUNCHES * len(shapes)
    # dispatch ids deliberately not in insertion order
    for j in reversed(range(n_cls)):
        rows.append((100 + j, _name(bench.CLASS_TMPL), "FETCH_SIZE", float(j), 0, 1))
    db = str(tmp_path / "k.db")
    _db(db, rows)
    g = bench.counter_dispatches(db, ("FETCH_SIZE",), v)
    assert [val["FETCH_SIZE"] for _, val in g["class"]] == [float(j) for j in range(n_cls)]
    pairs = bench.class_groups(g["class"], shapes)
    assert [k for k, _ in pairs] == [k for k, *_ in shapes]
    per = bench.PROBE_CLASS_LAUNCHES
    for i, (_, ds) in enumerate(pairs):
        assert [val["FETCH_SIZE"] for _, val in ds] == [float(per * i + r) for r in range(per)]
    # a launch missing: no class figures rather than shifted ones
    assert bench.class_groups(g["class"][1:], shapes) == []


def test_run_config_keeps_sizes_apart_from_options(bench):
    import argparse
    ns = argparse.Namespace(tokens=4096, hidden=None, overlap=False, chunk=0, layout="panel")
    cfg, chunk, default = bench.run_config(ns)
    assert (cfg["hidden"], cfg["dim"], cfg["n_cand"], chunk) == (12288, 3072, 96, 96)
    assert cfg["hidden_act"] == "f32" and default
    cfg, _, default = bench.run_config(argparse.Namespace(tokens=4096, hidden=None, overlap=True, chunk=0,
                                                          layout="panel"))
    assert cfg["hidden_act"] == "bf16" and cfg["hidden"] == 12288 and not default
    cfg, _, default = bench.run_config(argparse.Namespace(tokens=4096, hidden="bf16", overlap=False, chunk=0,
                                                          layout="panel"))
    assert not default and bench.gemm_variants(cfg)["gelu_mxfp4"][0] == "gemm_fp4_kernel<0, 3, 2>"


def test_power_sampler_without_amd_smi(bench, monkeypatch, tmp_path):
    monkeypatch.setenv("PATH", str(tmp_path))
    with bench.PowerSampler() as p:
        pass
    assert p.summary() is None


def test_power_sampler_is_off_under_a_profiler(bench, monkeypatch):
    # the profiler's preloaded library would initialise the GPU in each amd-smi child
    monkeypatch.setenv("LD_PRELOAD", "/opt/rocm/lib/librocprofiler-sdk-tool.so")
    assert bench.PowerSampler().cmd is None


def test_power_sampler_starts_a_python_script_with_this_interpreter(bench, monkeypatch, tmp_path):
    import sys
    script = tmp_path / "amd-smi"
    script.write_text("#!/usr/bin/env python3\nprint('{}')\n")
    script.chmod(0o755)
    monkeypatch.setenv("PATH", str(tmp_path))
    monkeypatch.delenv("LD_PRELOAD", raising=False)
    assert bench.PowerSampler().cmd == [sys.executable, str(script)]
