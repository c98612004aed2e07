"""bench.py's counter summaries, on small synthetic profiler databases (CPU).

The HBM-traffic and matrix-core-busy figures that bench.py reports come from
rocprofv3 results databases turned into committed summaries.  These tests
feed the summarizers a database with known counter values and check the
arithmetic: the copy-kernel scale factors, the per-dispatch means, the
cycles-per-shader-engine division, and that a summary taken on another
kernel source is ignored.
"""
import json
import os
import sqlite3

import pytest

import bench


def make_db(run_dir, rows):
    """rows: (kernel_name, counter_name, value), one row per dispatch."""
    os.makedirs(run_dir, exist_ok=True)
    con = sqlite3.connect(os.path.join(run_dir, "run_results.db"))
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?)", rows)
    con.commit()
    con.close()


COPY = "void at::native::vectorized_elementwise_kernel<8, at::native::neg_kernel>(int)"
K2 = "void lynx::(anonymous namespace)::gemm_sparse32<4>(unsigned short const*)"
K3 = "void lynx::(anonymous namespace)::gemm_dense32<4>(unsigned short const*)"


@pytest.fixture
def root(tmp_path, monkeypatch):
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def test_per_dispatch_mean(tmp_path):
    make_db(str(tmp_path / "d"), [(K2, "FETCH_SIZE", 10.0), (K2, "FETCH_SIZE", 30.0),
                                  (K3, "FETCH_SIZE", 7.0), (K2, "WRITE_SIZE", 99.0)])
    got = bench.per_dispatch_kib(str(tmp_path / "d"), "FETCH_SIZE")
    assert got == {K2: 20.0, K3: 7.0}


def test_traffic_scaled_by_the_copy_kernel(root):
    # the copy kernel reads and writes COPY_MIB MiB; its counters read half
    # the fetched bytes and all the written bytes, so the factors are 2 and 1
    mib = bench.COPY_MIB
    make_db(str(root / "f"), [(COPY, "FETCH_SIZE", mib * 512.0), (K2, "FETCH_SIZE", 1000.0),
                              (K2, "FETCH_SIZE", 3000.0)])
    make_db(str(root / "w"), [(COPY, "WRITE_SIZE", mib * 1024.0), (K2, "WRITE_SIZE", 500.0)])
    rec = bench.summarize_traffic(str(root / "f"), str(root / "w"), "unit")
    assert rec["copy_factor_fetch"] == pytest.approx(2.0)
    assert rec["copy_factor_write"] == pytest.approx(1.0)
    assert rec["fetch_bytes_per_launch"] == 2000 * 1024 * 2
    assert rec["write_bytes_per_launch"] == 500 * 1024
    assert rec["bytes_per_launch"] == 2000 * 1024 * 2 + 500 * 1024
    saved = json.load(open(root / "profiles" / "traffic_unit.json"))
    assert saved["kernel_sha"] == bench.source_sha("gemm_sparse32")
    # the bench line uses it while the kernel's sources are unchanged ...
    assert bench.traffic_for("unit") == rec["bytes_per_launch"]
    # ... and not once it was taken on other sources
    saved["kernel_sha"] = "0" * 16
    json.dump(saved, open(root / "profiles" / "traffic_unit.json", "w"))
    assert bench.traffic_for("unit") is None


def test_traffic_needs_exactly_one_matching_kernel(root):
    make_db(str(root / "f"), [(K2, "FETCH_SIZE", 1.0)])          # no copy kernel
    make_db(str(root / "w"), [(COPY, "WRITE_SIZE", 1.0), (K2, "WRITE_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_traffic(str(root / "f"), str(root / "w"), "unit")


def test_mfma_busy_fraction(root):
    # kernel cycles = SQ_BUSY_CYCLES / 32 shader engines; busy = matrix-core
    # busy cycles over (kernel cycles x 1024 SIMDs)
    kc = 200000.0
    make_db(str(root / "s"), [
        (K2, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * kc * 1024), (K2, "SQ_BUSY_CYCLES", kc * 32),
        (K2, "GRBM_GUI_ACTIVE", 8 * kc),
        (K3, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * kc * 1024), (K3, "SQ_BUSY_CYCLES", kc * 32),
        (COPY, "SQ_VALU_MFMA_BUSY_CYCLES", 0.0), (COPY, "SQ_BUSY_CYCLES", 5.0)])
    rec = bench.summarize_mfma(str(root / "s"), "unit")
    assert rec["kernels"]["gemm_sparse32<4>"]["mfma_busy"] == pytest.approx(0.5)
    assert rec["kernels"]["gemm_sparse32<4>"]["kernel_cycles"] == kc
    assert rec["kernels"]["gemm_dense32<4>"]["mfma_busy"] == pytest.approx(0.25)
    assert not any("neg" in k for k in rec["kernels"])           # no matrix work: left out
    assert bench.mfma_busy_for("unit") == {"gemm_sparse32<4>": 0.5, "gemm_dense32<4>": 0.25}
    # a kernel whose sources changed since is dropped; the others stay
    saved = json.load(open(root / "profiles" / "mfma_busy_unit.json"))
    saved["kernels"]["gemm_dense32<4>"]["source_sha"] = "0" * 16
    json.dump(saved, open(root / "profiles" / "mfma_busy_unit.json", "w"))
    assert bench.mfma_busy_for("unit") == {"gemm_sparse32<4>": 0.5}


def test_traffic_of_a_multi_layer_workload_is_per_step(root):
    """The block launches K2 once per sparse layer (both tile widths): the
    summary's per-step bytes are the mean per dispatch times the layers."""
    mib = bench.COPY_MIB
    K2n = K2.replace("<4>", "<3>")
    make_db(str(root / "f"), [(COPY, "FETCH_SIZE", mib * 512.0), (K2, "FETCH_SIZE", 100.0),
                              (K2n, "FETCH_SIZE", 300.0)])
    make_db(str(root / "w"), [(COPY, "WRITE_SIZE", mib * 1024.0), (K2, "WRITE_SIZE", 10.0),
                              (K2n, "WRITE_SIZE", 30.0)])
    rec = bench.summarize_traffic(str(root / "f"), str(root / "w"), "block")
    assert rec["launches_per_step"] == 4
    assert rec["bytes_per_step"] == (200 * 2 + 20) * 1024 * 4
    assert bench.traffic_for("block") == rec["bytes_per_step"]


def test_source_hash_covers_the_kernel_headers(monkeypatch, tmp_path):
    """Editing a header a kernel includes changes that kernel's hash."""
    for name in ("k_gemm.hip", "lynx_tile.h", "lynx_dma.h", "lynx_internal.h"):
        (tmp_path / name).write_text(name)
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    before = bench.source_sha("gemm_sparse32")
    (tmp_path / "lynx_tile.h").write_text("changed")
    assert bench.source_sha("gemm_sparse32") != before
    assert bench.source_sha("Cijk_library_kernel") is None


def test_report_renders_one_row_per_record(tmp_path):
    """--report: the last benchmark line of each file becomes one table row,
    times in µs, ratios with two decimals, missing counters as a dash."""
    rec = {"metric": "m", "value": 1456.2, "ms_per_step": 0.218, "ms_per_step_after_idle": 0.23,
           "config": {"workload": "mlp_up: X[4096x3072] -> Y[4096x12288]"},
           "interleaved_ms": {"sparse_layer": 0.19026, "dense_layer": 0.27192, "torch_matmul": 0.22773},
           "split_ms": {"sparsify": 0.01745, "sparse_gemm_lora": 0.17202},
           "speedup_vs_dense": 1.429, "speedup_vs_torch_matmul": 1.197, "speedup_vs_best_dense": 1.197,
           "roofline": {"frac": 0.3721}, "sparsify_roofline": {"frac": 0.2884},
           "mfma_busy": {"gemm_dense32<4>": 0.716, "gemm_sparse32<4>": 0.5996},
           "cpu_baseline": {"value": 0.2371, "cores": 16}}
    other = dict(rec, config={"workload": "tiny: ..."}, mfma_busy=None, cpu_baseline=None)
    del other["ms_per_step_after_idle"]
    a, b = tmp_path / "a.json", tmp_path / "b.json"
    a.write_text("warm-up noise\n" + json.dumps(dict(rec, value=1.0)) + "\n" + json.dumps(rec) + "\n")
    b.write_text(json.dumps(other) + "\n")
    table = bench.render_report(bench.read_records([str(a), str(b)])).splitlines()
    assert len(table) == 4 and table[1].count("---") == len(bench.REPORT_COLUMNS)
    row = [c.strip() for c in table[2].strip("|").split("|")]
    assert row == ["mlp_up", "1456", "0.2180", "0.2300", "190.3", "271.9", "227.7", "1.43×", "1.20×", "1.20×",
                   "17.4", "172.0", "0.372", "0.60", "0.288", "0.237 (16 threads)"]
    tiny = [c.strip() for c in table[3].strip("|").split("|")]
    assert tiny[0] == "tiny" and tiny[13] == "—" and tiny[15] == "—"
    (tmp_path / "none.json").write_text("no record\n")
    with pytest.raises(SystemExit):
        bench.read_records([str(a), str(tmp_path / "none.json")])


def test_power_sampler_reads_hwmon_and_sclk(tmp_path):
    """--sustained's sampler: board power from hwmon (µW) and the starred
    shader-clock level of pp_dpm_sclk; missing files give nulls."""
    (tmp_path / "power1_input").write_text("750000000\n")
    (tmp_path / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 1500Mhz *\n2: 2400Mhz\n")
    ps = bench.PowerSampler(period_s=0.001)
    ps.power_path, ps.sclk_path, ps.cap_w = str(tmp_path / "power1_input"), str(tmp_path / "pp_dpm_sclk"), 1400.0
    ps.start()
    import time
    time.sleep(0.05)
    out = ps.stop()
    assert out["power_w"]["mean"] == 750.0 and out["power_w"]["samples"] > 0
    assert out["sclk_mhz"]["mean"] == 1500 and out["power_cap_w"] == 1400.0
    empty = bench.PowerSampler()
    empty.power_path = empty.sclk_path = None
    empty.start()
    assert empty.stop()["power_w"] is None
