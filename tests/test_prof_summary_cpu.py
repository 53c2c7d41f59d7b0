"""CPU tests of the rocprofv3 summariser on small hand-made CSV files: only
dispatches that start inside a workload's timed window count, per-kernel
averages and per-step counts, the copy-calibrated HBM bytes, the traffic
table keyed by workload and kind, and the per-dispatch MFMA counter sums."""
import csv
import json
import os

import pytest

from speculative_decoding_encoder_amd import prof_summary as ps

GEMM = "void wf::gemm_rk_kernel<1, 1, 1, 5, false>(wf::GemmArgs)"
PREP = "wf::prepare_kernel(wf::PrepArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _log(path, wins):
    with open(path, "w") as f:
        f.write("[bench] inputs generated in 1.0s\n")
        for what, t0, t1 in wins:
            f.write(f"[bench] timed-window {what} {t0} {t1}\n")


def _csv(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_short_name_and_windows(tmp_path):
    assert ps.short_name('"' + GEMM + '"') == "wf::gemm_rk_kernel<1, 1, 1, 5, false>"
    assert ps.short_name(PREP) == "wf::prepare_kernel"
    assert ps.short_name(COPY) == COPY
    log = tmp_path / "a.log"
    _log(log, [("wl-a", 100, 200), ("wl-b", 300, 400), ("wl-a", 500, 600)])
    w = ps.windows(str(log))
    assert w == {"wl-a": [(100, 200), (500, 600)], "wl-b": [(300, 400)]}
    assert ps.in_window({"Start_Timestamp": "200"}, w["wl-a"])
    assert not ps.in_window({"Start_Timestamp": "250"}, w["wl-a"])


def test_stats_keeps_the_timed_window_only(tmp_path):
    log = tmp_path / "tr.log"
    _log(log, [("wl", 1000, 30000)])
    # two timed steps (ns): a prepare of 2 us and GEMMs of 3 and 5 us; the
    # second step's last GEMM starts inside the window and ends after it (8.3 us)
    rows = []
    for t in (1000, 12000):
        rows.append({"Kernel_Name": PREP, "Start_Timestamp": t, "End_Timestamp": t + 2000})
        rows.append({"Kernel_Name": GEMM, "Start_Timestamp": t + 2100, "End_Timestamp": t + 5100})
        rows.append({"Kernel_Name": GEMM, "Start_Timestamp": t + 5200, "End_Timestamp": t + 10200})
    rows[-1]["Start_Timestamp"], rows[-1]["End_Timestamp"] = 29900, 38200
    # warm-up and later dispatches outside the window: a 1 ms GEMM, a prepare
    rows.append({"Kernel_Name": GEMM, "Start_Timestamp": 10, "End_Timestamp": 1_000_010})
    rows.append({"Kernel_Name": PREP, "Start_Timestamp": 31000, "End_Timestamp": 32000})
    _csv(str(tmp_path / "run" / "x" / "run_kernel_trace.csv"),
         ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    out = tmp_path / "s.txt"
    ps.main(["stats", "--dir", str(tmp_path / "run"), "--log", str(log), "--window", "wl",
             "--title", "t", "--command", "c", "--out", str(out)])
    text = out.read_text()
    assert "2 graph-replayed fixed-block steps, 6 dispatches" in text
    assert len([l for l in text.splitlines() if l.startswith("wf::")]) == 2
    gemm = next(l for l in text.splitlines() if l.startswith("wf::gemm_rk_kernel"))
    prep = next(l for l in text.splitlines() if l.startswith("wf::prepare_kernel"))
    g = gemm.split()[-6:]
    p = prep.split()[-6:]
    # calls, per step, avg, min, max, pct
    assert g[0] == "4" and float(g[1]) == 2.0
    assert float(g[2]) == pytest.approx((3 + 5 + 3 + 8.3) / 4, abs=0.01)
    assert float(g[3]) == pytest.approx(3.0) and float(g[4]) == pytest.approx(8.3)
    assert p[0] == "2" and float(p[2]) == pytest.approx(2.0)
    total = 3 + 5 + 3 + 8.3 + 4
    assert float(g[5]) == pytest.approx(100 * 19.3 / total, abs=0.01)
    assert f"summed kernel time {total / 2:.1f} us per step" in text
    assert f"# {(38200 - 1000) / 1e3 / 2:.1f} us per step" in text   # first start to last end


def test_stats_refuses_a_missing_window(tmp_path):
    log = tmp_path / "tr.log"
    _log(log, [("other", 0, 10)])
    _csv(str(tmp_path / "run" / "k_kernel_trace.csv"),
         ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
         [{"Kernel_Name": PREP, "Start_Timestamp": 1, "End_Timestamp": 2}])
    with pytest.raises(SystemExit):
        ps.main(["stats", "--dir", str(tmp_path / "run"), "--log", str(log), "--window", "wl",
                 "--title", "t", "--command", "c"])


def _counter_run(root, name, counter, copy_kib, kernel_kib):
    """A counter run: the calibration copy inside its window, the kernel
    twice inside the workload's window and once outside it."""
    log = root / f"{name}.log"
    _log(log, [("calibration-copy", 10, 20), ("wl", 100, 200)])
    rows = [
        {"Kernel_Name": COPY, "Start_Timestamp": 12, "Counter_Name": counter,
         "Counter_Value": copy_kib, "Dispatch_Id": 1},
        {"Kernel_Name": COPY, "Start_Timestamp": 15, "Counter_Name": counter,
         "Counter_Value": copy_kib / 4, "Dispatch_Id": 2},          # a smaller copy
        {"Kernel_Name": GEMM, "Start_Timestamp": 110, "Counter_Name": counter,
         "Counter_Value": kernel_kib[0], "Dispatch_Id": 3},
        {"Kernel_Name": GEMM, "Start_Timestamp": 150, "Counter_Name": counter,
         "Counter_Value": kernel_kib[1], "Dispatch_Id": 4},
        {"Kernel_Name": GEMM, "Start_Timestamp": 300, "Counter_Name": counter,
         "Counter_Value": 1e9, "Dispatch_Id": 5},                   # after the window
        {"Kernel_Name": PREP, "Start_Timestamp": 120, "Counter_Name": counter,
         "Counter_Value": 1e9, "Dispatch_Id": 6},                   # another kernel
    ]
    _csv(str(root / name / "r_counter_collection.csv"),
         ["Kernel_Name", "Start_Timestamp", "Counter_Name", "Counter_Value", "Dispatch_Id"], rows)
    return str(root / name), str(log)


def test_traffic_scales_by_the_copy_and_keys_the_table(tmp_path):
    mib = 256.0 * 2 ** 20
    # the copy: FETCH_SIZE reads half its bytes, WRITE_SIZE all of them
    fd, fl = _counter_run(tmp_path, "fetch", "FETCH_SIZE", mib / 1024 / 2, (1000.0, 2000.0))
    wd, wl = _counter_run(tmp_path, "write", "WRITE_SIZE", mib / 1024, (40.0, 60.0))
    table = tmp_path / "t.json"
    table.write_text(json.dumps([{"workload": "wl", "kind": "oproj", "stale": True},
                                 {"workload": "other", "kind": "oproj"}]))
    args = ["traffic", "--fetch-dir", fd, "--fetch-log", fl, "--write-dir", wd, "--write-log", wl,
            "--window", "wl", "--kind", "oproj", "--symbol", "wf::gemm_rk_kernel<1,",
            "--command", "c", "--algo-bytes", "3000000", "--json", str(table),
            "--out", str(tmp_path / "o.txt")]
    ps.main(args)
    ps.main(args)                                   # a second run replaces its entry
    entries = json.loads(table.read_text())
    assert [(e["workload"], e["kind"]) for e in entries] == [("other", "oproj"), ("wl", "oproj")]
    e = entries[1]
    assert e["dispatches"] == 2 and "stale" not in e
    assert e["fetch_scale"] == pytest.approx(2.0) and e["write_scale"] == pytest.approx(1.0)
    assert e["fetch_kib_avg"] == pytest.approx(1500.0) and e["write_kib_avg"] == pytest.approx(50.0)
    assert e["hbm_bytes_per_launch"] == pytest.approx((1500.0 * 2 + 50.0) * 1024)
    assert e["source_hash"] == ps.kernel_source_hash("wl")
    text = (tmp_path / "o.txt").read_text()
    assert f"HBM bytes per launch: {3050 * 1024 / 1e6:.3f} MB" in text
    assert f"traffic / algorithmic {3050 * 1024 / 3e6:.3f}" in text


def test_mfma_sums_counters_per_dispatch(tmp_path):
    log = tmp_path / "m.log"
    _log(log, [("wl", 100, 200)])
    rows = []
    for d, (util, bf, f16) in enumerate([(20.0, 3e9, 1e9), (30.0, 5e9, 1e9)]):
        for name, v in (("MfmaUtil", util), ("MfmaFlopsBF16", bf), ("MfmaFlopsF16", f16)):
            rows.append({"Kernel_Name": GEMM, "Start_Timestamp": 110 + d, "Counter_Name": name,
                         "Counter_Value": v, "Dispatch_Id": d})
    rows.append({"Kernel_Name": GEMM, "Start_Timestamp": 500, "Counter_Name": "MfmaUtil",
                 "Counter_Value": 99.0, "Dispatch_Id": 9})
    rows.append({"Kernel_Name": PREP, "Start_Timestamp": 120, "Counter_Name": "MfmaUtil",
                 "Counter_Value": 0.0, "Dispatch_Id": 7})
    _csv(str(tmp_path / "run" / "r_counter_collection.csv"),
         ["Kernel_Name", "Start_Timestamp", "Counter_Name", "Counter_Value", "Dispatch_Id"], rows)
    out = tmp_path / "m.txt"
    ps.main(["mfma", "--dir", str(tmp_path / "run"), "--log", str(log), "--window", "wl",
             "--title", "t", "--command", "c", "--out", str(out)])
    lines = [l for l in out.read_text().splitlines() if l.startswith("wf::")]
    assert len(lines) == 1                          # no flops: the prepare kernel is left out
    f = lines[0].split()
    assert f[-3] == "2" and float(f[-2]) == pytest.approx(25.0) and float(f[-1]) == pytest.approx(5.0)
