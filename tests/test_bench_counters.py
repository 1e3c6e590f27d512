"""Host logic of the measurement path (no GPU): the rocprofv3 counter summary
that becomes the bench's `traffic` figure, and the source-hash gate that
drops it once a kernel changes.  The counter CSVs are synthetic, with
figures worked out by hand below."""
import csv
import json
import os

import bench

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(dirpath, counter, dispatches):
    """dispatches: [(kernel name, [values of the rows of that dispatch])]."""
    os.makedirs(dirpath, exist_ok=True)
    with open(os.path.join(dirpath, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, values) in enumerate(dispatches):
            for v in values:
                w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})
            # another counter in the same file is ignored
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": "GRBM_COUNT", "Counter_Value": 1e9})


def _runs(tmp_path, write_gemv_calls=2):
    copy = "__amd_rocclr_copyBuffer"
    mib = bench.COPY_MIB * 1024  # KiB of one calibration copy
    fetch = [
        ("void stq::gemv_kernel<1>(KArgs)", [500.0, 500.0]),       # one dispatch over two rows: 1000 KiB
        ("stq::reduce_splits_kernel(...)", [100.0]),
        ("void stq::gemv_kernel<1>(KArgs)", [1000.0]),
        ("stq::reduce_splits_kernel(...)", [100.0]),
        ("stq::grouped_gemm_kernel(GArgs)", [5000.0]),
        ("some_other_kernel", [7.0]),
        (copy, [mib / 4, mib / 4]),                                # reads as half its size: factor 2
        (copy, [mib / 2]),
        (copy, [16.0]),                                            # a small copy: not a calibration copy
    ]
    write = [("void stq::gemv_kernel<1>(KArgs)", [10.0])] * write_gemv_calls + [
        ("stq::reduce_splits_kernel(...)", [50.0]),
        ("stq::reduce_splits_kernel(...)", [50.0]),
        ("stq::grouped_gemm_kernel(GArgs)", [2000.0]),
        (copy, [float(mib)]),                                      # factor 1
    ]
    _write(tmp_path / "fetch", "FETCH_SIZE", fetch)
    _write(tmp_path / "write", "WRITE_SIZE", write)
    return str(tmp_path / "fetch"), str(tmp_path / "write")


def test_counter_summary_scales_and_averages_per_call(tmp_path, monkeypatch):
    out = tmp_path / "hbm_counters.json"
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(out))
    assert bench.summarise_counters(*_runs(tmp_path)) == 0
    d = json.loads(out.read_text())
    g = d["k_gemv.hip"]
    # GEMV + reduction: fetch (1000 + 1000 + 100 + 100) KiB x 2 / 2 calls, write (10 + 10 + 50 + 50) KiB x 1 / 2
    assert g["calls"] == 2
    assert g["fetch_bytes_per_call"] == 2200 * 1024
    assert g["write_bytes_per_call"] == 60 * 1024
    assert g["bytes_per_launch"] == 2260 * 1024
    assert g["scale_factors"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    assert g["source_hash"] == bench.kernel_source_hash("k_gemv.hip")
    m = d["k_gemm.hip"]
    assert (m["calls"], m["fetch_bytes_per_call"], m["write_bytes_per_call"]) == (1, 5000 * 1024 * 2, 2000 * 1024)


def test_counter_summary_refuses_mismatched_runs(tmp_path, monkeypatch):
    out = tmp_path / "hbm_counters.json"
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(out))
    assert bench.summarise_counters(*_runs(tmp_path, write_gemv_calls=3)) == 1
    assert not out.exists()


def test_traffic_is_reported_only_for_the_counted_source(tmp_path, monkeypatch):
    out = tmp_path / "hbm_counters.json"
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(out))
    assert bench.measured_traffic("k_gemv.hip") is None  # no counters taken
    out.write_text(json.dumps({"k_gemv.hip": {"source_hash": bench.kernel_source_hash("k_gemv.hip"),
                                              "bytes_per_launch": 123}}))
    assert bench.measured_traffic("k_gemv.hip") == 123
    out.write_text(json.dumps({"k_gemv.hip": {"source_hash": "0" * 16, "bytes_per_launch": 123}}))
    assert bench.measured_traffic("k_gemv.hip") is None  # the kernel changed since



def test_trace_summary_drops_warmup_dispatches(tmp_path, capsys):
    """Kernels called once or eight times per step: the timed mean leaves out
    the warm-up steps' dispatches (the first ones by start time, whatever the
    row order); a kernel called at no multiple of the step count (setup) has
    no timed figure."""
    d = tmp_path / "trace"
    d.mkdir()
    rows, t = [], 0
    for step in range(7):                                  # 2 warm-up + 5 timed steps
        for _ in range(8):
            rows.append(("void stq::gemv_kernel<1, false>(KArgs)", t, t + 100_000 + 1000 * step))
            t += 200_000
        rows.append(("stq::grouped_gemm_kernel(GArgs)", t, t + (2_000_000 if step < 2 else 1_000_000)))
        t += 3_000_000
    rows.append(("setup_kernel", 5, 10))
    rows.reverse()
    with open(d / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, b, e in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": b, "End_Timestamp": e})
    assert bench.summarise_trace(str(d), warmup=2, steps=5) == 0
    out = capsys.readouterr().out
    gemm = next(l for l in out.splitlines() if "grouped_gemm" in l).split("|")
    assert [c.strip() for c in gemm[2:8]] == ["7", "5", "1000.0", "1000.0", "1000.0", "1285.7"]
    gemv = next(l for l in out.splitlines() if "gemv_kernel" in l).split("|")
    assert [c.strip() for c in gemv[2:5]] == ["56", "40", "104.0"]   # steps 2..6: 102..106 us
    setup = next(l for l in out.splitlines() if "setup_kernel" in l).split("|")
    assert setup[3].strip() == "-"
