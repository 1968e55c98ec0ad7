"""Host logic of bench.py (no GPU): the one-GPU contract and the rocprofv3
counter records that give the roofline its HBM traffic."""

import importlib.util
import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _counter_db(path, counter, rows):
    """A database shaped like rocprofv3's: one row per (dispatch, counter instance)."""
    c = sqlite3.connect(path)
    c.execute("create table counters_collection (kernel_name text, counter_name text, value real, "
              "duration integer, dispatch_id integer)")
    c.executemany("insert into counters_collection values (?, ?, ?, 0, ?)",
                  [(k, counter, v, d) for k, v, d in rows])
    c.commit()
    c.close()


def test_traffic_record_scales_by_the_copy_calibration(bench, tmp_path):
    kname = "void " + bench.DOMINANT["dense"][0] + "(fp8bs::GemmArgs)"
    copy = "__amd_rocclr_copyBuffer"
    gib_kib = bench.COPY_BYTES / 1024
    # the copy's 1 GiB reads as half in FETCH_SIZE and in full in WRITE_SIZE; counter values of one
    # dispatch are split over two instances (summed), and two dispatches are averaged
    _counter_db(tmp_path / "f.db", "FETCH_SIZE",
                [(copy, gib_kib / 4, 1), (copy, gib_kib / 4, 1), (kname, 600.0, 2), (kname, 400.0, 2),
                 (kname, 1500.0, 3), (kname, 500.0, 3)])
    _counter_db(tmp_path / "w.db", "WRITE_SIZE",
                [(copy, gib_kib, 1), (kname, 300.0, 2), (kname, 300.0, 3)])
    rec = bench.summarize_pmc(str(tmp_path / "f.db"), str(tmp_path / "w.db"), "dense", "test command",
                              out=str(tmp_path / "rec.json"))
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["launches"] == [2, 2]
    # mean of (1000, 2000) KiB fetched, x2; 300 KiB written, x1
    assert rec["hbm_fetch_bytes_per_launch"] == pytest.approx(1500 * 1024 * 2.0)
    assert rec["hbm_write_bytes_per_launch"] == pytest.approx(300 * 1024)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(1500 * 1024 * 2 + 300 * 1024)
    assert json.load(open(tmp_path / "rec.json")) == rec


def test_moe_record_sums_each_gate_up_call(bench, tmp_path):
    """The MoE record takes the grouped gate+up call (table + 256-row pass +
    short-tile pass after the activation quantizer), not the down call that
    follows the gated activation."""
    copy = "__amd_rocclr_copyBuffer"
    gib_kib = bench.COPY_BYTES / 1024
    seq = ["void fp8bs::quant_w_kernel<0>(fp8bs::QWArgs)", "void fp8bs::quant_act_kernel<0>(...)",
           "void fp8bs::grouped_tile_table_kernel<256, 128>(...)",
           "void fp8bs::gemm_dma_kernel<256, 256, 4, 2, false, true, false, false, false>(fp8bs::GemmArgs)",
           "void fp8bs::gemm_dma_kernel<128, 256, 2, 4, false, true, false, false, false>(fp8bs::GemmArgs)",
           "void fp8bs::swiglu_quant_kernel<0>(...)",
           "void fp8bs::grouped_tile_table_kernel<256, 128>(...)",
           "void fp8bs::gemm_dma_kernel<256, 256, 4, 2, false, true, false, false, false>(fp8bs::GemmArgs)",
           "void fp8bs::gemm_dma_kernel<128, 256, 2, 4, false, true, false, false, false>(fp8bs::GemmArgs)"]
    vals = [1000.0, 100.0, 1.0, 500.0, 50.0, 70.0, 2.0, 300.0, 30.0]
    rows, d = [], 0
    for step in range(2):  # two steps; the second gate+up call moves 2x as much
        for k, v in zip(seq, vals):
            d += 1
            rows.append((k, v * (1 + step), d))
    _counter_db(tmp_path / "f.db", "FETCH_SIZE", rows + [(copy, gib_kib / 2, d + 1)])
    _counter_db(tmp_path / "w.db", "WRITE_SIZE", rows + [(copy, gib_kib, d + 1)])
    rec = bench.summarize_pmc(str(tmp_path / "f.db"), str(tmp_path / "w.db"), "moe", "test command",
                              out=str(tmp_path / "rec.json"))
    assert rec["launches"] == [2, 2]
    per_call = (1.0 + 500.0 + 50.0) * 1.5  # mean over the two steps
    assert rec["hbm_fetch_bytes_per_launch"] == pytest.approx(per_call * 1024 * 2.0)
    assert rec["hbm_write_bytes_per_launch"] == pytest.approx(per_call * 1024)


def test_no_kernel_in_the_database_is_an_error(bench, tmp_path):
    _counter_db(tmp_path / "f.db", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 1.0, 1)])
    _counter_db(tmp_path / "w.db", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1.0, 1)])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(tmp_path / "f.db"), str(tmp_path / "w.db"), "dense", "c",
                            out=str(tmp_path / "rec.json"))


def test_traffic_is_withheld_once_the_kernel_source_changed(bench, tmp_path, monkeypatch):
    kprefix, src, fname = bench.DOMINANT["dense"]
    rec = {"hbm_bytes_per_launch": 123.0, "source_sha256_16": bench.src_hash(src)}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / fname).write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_for("dense") == (123.0, "profiles/" + fname)
    rec["source_sha256_16"] = "0" * 16
    (tmp_path / "profiles" / fname).write_text(json.dumps(rec))
    value, why = bench.traffic_for("dense")
    assert value is None and why.startswith("stale")
    assert bench.traffic_for("decode") == (None, None)


def test_kernel_timer_median_and_min():
    """Per-kernel median and min of the timed launches (fake events stand in for HIP events)."""
    import bench

    class Ev:
        def __init__(self, t):
            self.t = t

        def elapsed_time(self, other):
            return other.t - self.t

    kt = bench.KernelTimer()
    kt.pairs["k"] = [(Ev(0.0), Ev(d)) for d in (3.0, 1.0, 2.0, 10.0)]
    assert kt.avg_ms("k") == 4.0
    assert kt.spread("k") == (2.5, 1.0)
    kt.pairs["odd"] = [(Ev(1.0), Ev(1.0 + d)) for d in (5.0, 4.0, 6.0)]
    assert kt.spread("odd") == (5.0, 4.0)


def test_roofline_helpers(bench):
    r = bench.roof_hbm("k", 1.0, 4e9)
    assert r["bound"] == "hbm" and r["achieved"] == pytest.approx(4000.0) and r["frac"] == pytest.approx(0.5)
    r = bench.roof_mfma("k", 1.0, 2.5e12)
    assert r["bound"] == "mfma" and r["frac"] == pytest.approx(0.5)
    # the bound that binds: bytes at 8 TB/s against FLOPs at 5 PFLOP/s
    assert bench.roof_binding("k", 1.0, 1e12, 1e9)["bound"] == "mfma"   # 200 us of MFMA vs 125 us of HBM
    assert bench.roof_binding("k", 1.0, 1e11, 1e9)["bound"] == "hbm"


@pytest.mark.parametrize("name", ["cpu_recal", "cpu_quant_act", "cpu_dense", "cpu_decode", "cpu_moe", "cpu_tiny",
                                  "cpu_attention"])
def test_cpu_baselines_run(bench, name):
    """Every row's oracle baseline runs on the host and reports both thread counts."""
    kw = {"target_s": 0.01}
    if name == "cpu_moe":
        kw["experts"] = 2
    cb = getattr(bench, name)(**kw)
    assert cb["kind"] == "oracle" and cb["cores"] >= 1
    assert cb["value"] > 0 and cb["value_1thread"] > 0
    assert isinstance(cb["sample"], str) and isinstance(cb["sample_1thread"], str)
    import oracle
    assert oracle.max_threads() == cb["cores"]   # the thread count is restored
