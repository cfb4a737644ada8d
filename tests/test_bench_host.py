"""Host logic of bench.py and of the binding, on the CPU: the one-GPU
guard, the calibration of rocprofv3 byte counters against a copy of known
size, the kernel-statistics summary, and the loud failure of the binding
when the HIP library is missing (there is no CPU fallback)."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import kv_cache_block_amd as kka

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GIB_KIB = float(1 << 20)  # 1 GiB in KiB


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_counter_summary_calibrates_against_the_copy(tmp_path):
    """The copy of 1 GiB reads as 2 GiB of FETCH_SIZE (factor 0.5) and
    1 GiB of WRITE_SIZE (factor 1); every kernel's KiB are scaled by those
    factors and averaged over its dispatches."""
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    pool = "void kka::(anonymous namespace)::pool_kernel<0, 256>(kka::PoolArgs)"
    score = "void kka::(anonymous namespace)::score_topk_kernel<256, 8, 4, 4, 4, false>(kka::ScoreArgs, float*)"
    small = "void kka::(anonymous namespace)::score_topk_kernel<1024, 8, 4, 2, 2, false>(kka::ScoreArgs, float*)"
    copy = "__amd_rocclr_copyBuffer"
    fetch = [[copy, 1 << 20, "FETCH_SIZE", 2 * GIB_KIB], [copy, 64, "FETCH_SIZE", 1.0],
             [pool, 2097152, "FETCH_SIZE", 1000.0], [pool, 2097152, "FETCH_SIZE", 3000.0],
             [score, 1146880, "FETCH_SIZE", 400.0], [small, 36864, "FETCH_SIZE", 40.0],
             [pool, 2097152, "OTHER", 9e9]]
    write = [[copy, 1 << 20, "WRITE_SIZE", GIB_KIB], [copy, 64, "WRITE_SIZE", 1.0],
             [pool, 2097152, "WRITE_SIZE", 10.0], [pool, 2097152, "WRITE_SIZE", 30.0],
             [score, 1146880, "WRITE_SIZE", 8.0], [small, 36864, "WRITE_SIZE", 2.0]]
    fcsv, wcsv = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write_csv(fcsv, hdr, fetch)
    _write_csv(wcsv, hdr, write)
    bench.write_counter_summary(str(fcsv), str(wcsv), str(tmp_path), command="cmd")
    k = json.load(open(tmp_path / os.path.basename(bench.COUNTERS)))
    assert k["fetch_factor"] == 0.5 and k["write_factor"] == 1.0
    # pool: mean fetch 2000 KiB * 0.5 = 1,024,000 B; mean write 20 KiB = 20,480 B
    assert k["traffic_bytes_per_launch"] == 1024000 + 20480
    assert k["per_kernel"]["pool_kernel<0, 256> grid=2097152"] == {"fetch_bytes": 1024000, "write_bytes": 20480,
                                                                   "dispatches": 2}
    assert k["kernel_source_sha256_16"] == bench.kernel_source_hash("kka_pool.hip")
    assert k["commands"] == "cmd"
    s = json.load(open(tmp_path / os.path.basename(bench.SCORE_COUNTERS)))
    # the serving call (the large one-launch grid): 400 KiB * 0.5 + 8 KiB; the one-sequence launch is not it
    assert s["traffic_bytes_per_call"] == 204800 + 8192
    assert s["kernel_source_sha256_16"] == bench.kernel_source_hash("kka_score.hip")


def test_pool_counter_summary_of_a_reported_workload(tmp_path):
    """The 0.5B K-pool's counter pass: bytes per call from the same copy
    calibration, beside the workload's algorithmic bytes."""
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    pool = "void kka::(anonymous namespace)::pool_kernel<0, 256>(kka::PoolArgs)"
    copy = "__amd_rocclr_copyBuffer"
    fetch = [[copy, 1 << 20, "FETCH_SIZE", 2 * GIB_KIB], [pool, 65536, "FETCH_SIZE", 49000.0],
             [pool, 65536, "FETCH_SIZE", 51000.0]]
    write = [[copy, 1 << 20, "WRITE_SIZE", GIB_KIB], [pool, 65536, "WRITE_SIZE", 64.0],
             [pool, 65536, "WRITE_SIZE", 64.0]]
    fcsv, wcsv = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write_csv(fcsv, hdr, fetch)
    _write_csv(wcsv, hdr, write)
    out = tmp_path / "c1.json"
    bench.write_ragged_counter_summary(str(fcsv), str(wcsv), "-", str(out), command="cmd", which="c1")
    k = json.load(open(out))
    # mean fetch 50,000 KiB * 0.5, mean write 64 KiB
    assert k["traffic_bytes_per_call"] == 25_600_000 + 65_536
    assert k["kpool_algorithmic_bytes"] == 25_232_384
    assert k["traffic_over_algorithmic"] == round((25_600_000 + 65_536) / 25_232_384, 5)
    assert k["per_kernel"]["pool_kernel<0, 256> grid=65536"]["dispatches"] == 2
    assert k["kernel_source_sha256_16"] == bench.kernel_source_hash("kka_pool.hip")
    assert "0.5B" in k["workload"]


def test_counter_summary_needs_the_copy(tmp_path):
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    rows = [["void kka::(anonymous namespace)::pool_kernel<0, 256>(kka::PoolArgs)", 2097152, "FETCH_SIZE", 1.0]]
    _write_csv(tmp_path / "f.csv", hdr, rows)
    _write_csv(tmp_path / "w.csv", hdr, [[r[0], r[1], "WRITE_SIZE", 1.0] for r in rows])
    with pytest.raises(SystemExit, match="copy"):
        bench.write_counter_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path), command="")


def test_stats_summary_tables(tmp_path):
    """The statistics table in the profiler's order, and per launch shape
    (kernel, grid, work-group) the count, mean, median and minimum of the
    traced durations of the library's kernels."""
    stats = tmp_path / "bench_kernel_stats.csv"
    _write_csv(stats, ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
               [["void kka::(anonymous namespace)::pool_kernel<0, 256>(kka::PoolArgs)", 3, 5000, 1000, 8000, 90.5],
                ["at::native::fill", 1, 250, 250, 250, 9.5]])
    pk = "void kka::(anonymous namespace)::pool_kernel<0, 256>(kka::PoolArgs)"
    trace_rows = [[pk, 2097152, 256, 0, 8000], [pk, 2097152, 256, 10000, 16000], [pk, 458752, 256, 20000, 21000],
                  ["at::native::fill", 64, 64, 0, 250]]
    _write_csv(tmp_path / "bench_kernel_trace.csv",
               ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"], trace_rows)
    out = tmp_path / "s.md"
    bench.write_stats_summary(str(stats), str(out), "Title", command="rocprofv3 -- python bench.py")
    text = out.read_text().splitlines()
    assert text[0] == "# Title"
    assert "rocprofv3 -- python bench.py" in text
    assert "| `pool_kernel<0, 256>` | 3 | 5.00 | 1.00 | 8.00 | 90.50 |" in text
    assert "| `at::native::fill` | 1 | 0.25 | 0.25 | 0.25 | 9.50 |" in text
    # per shape: 8 and 6 us (mean 7, upper median 8, min 6), then the 1 us launch; torch's kernel left out
    assert "| `pool_kernel<0, 256>` | 2097152 | 256 | 2 | 7.00 | 8.00 | 6.00 |" in text
    assert "| `pool_kernel<0, 256>` | 458752 | 256 | 1 | 1.00 | 1.00 | 1.00 |" in text
    assert not any(line.startswith("| `at::native::fill` | 64") for line in text)


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kka, "LIB_PATH", str(tmp_path / "libkka.so"))
    monkeypatch.setattr(kka, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        kka.lib()


def test_cpu_baseline_fields_on_a_small_workload():
    """The oracle leg of the benchmark on a reduced 7B-shape sequence (256
    blocks of 16 tokens, 2 layers): whole-step rate, per-step time and the
    decode-step part timed alone."""
    import synth
    w = synth.config3(0, n_blocks=256, L=2)
    step_bytes = 256 * 16 * 2 * w.H * w.D * 2
    cb = bench.cpu_baseline(w, step_bytes, 0.2)
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["unit"] == "GB/s"
    assert cb["value"] > 0 and cb["ms_per_step"] > 0 and cb["levels_score_topk_ms_per_step"] > 0
    assert cb["levels_score_topk_ms_per_step"] < cb["ms_per_step"]
