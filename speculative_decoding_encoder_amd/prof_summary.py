"""Summaries of rocprofv3 runs of bench.py, cut to the timed steady state.

bench.py --mark-timed prints, per workload, the host-clock window
(CLOCK_MONOTONIC ns, the clock of rocprofv3's timestamps) of its timed
fixed-block replays and of the calibration copies. This module reads the
rocprofv3 CSV output of a kernel-trace run or of a counter run and keeps the
dispatches that start inside such a window.

  python -m speculative_decoding_encoder_amd.prof_summary stats \\
      --dir RUN_DIR --log BENCH_LOG \\
      --window large-v3-verify-b32-greedy --title "..." --command "..." --out FILE

  python -m speculative_decoding_encoder_amd.prof_summary mfma --dir D --log L \\
      --window WORKLOAD --title "..." --command "..." --out FILE

  python -m speculative_decoding_encoder_amd.prof_summary traffic \\
      --fetch-dir D1 --fetch-log L1 --write-dir D2 --write-log L2 \\
      --window WORKLOAD --kind oproj --symbol 'wf::gemm_rk_kernel<1,' \\
      --algo-bytes 3276800 --command "..." --out FILE --json profiles/hbm_traffic.json

Traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) averaged over the
kernel's dispatches in the window, each scaled by what the same counter reads
for the largest calibration copy (a device-to-device copy of known size:
bytes read = bytes written = its size).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from typing import Dict, List, Optional, Tuple

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_decoding_encoder_amd", "csrc")
ENCODER_SOURCES = ("encoder.hip", "wf_device.h")
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def is_encoder_workload(workload: str) -> bool:
    return "encoder" in workload


def kernel_source_hash(workload: str = "") -> str:
    """sha256 over the kernel sources of a workload, in name order: the
    encoder's (encoder.hip and the device helpers) for an encoder workload,
    every other csrc/*.hip and csrc/*.h for the verify path."""
    enc = is_encoder_workload(workload)
    hsh = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if not name.endswith((".hip", ".h")):
            continue
        if enc and name not in ENCODER_SOURCES:
            continue
        if not enc and name == "encoder.hip":
            continue
        with open(os.path.join(CSRC, name), "rb") as f:
            hsh.update(name.encode() + b"\0" + f.read())
    return hsh.hexdigest()[:16]


def windows(log_path: str) -> Dict[str, List[Tuple[int, int]]]:
    """[bench] timed-window <what> <t0> <t1> lines of a bench log."""
    out: Dict[str, List[Tuple[int, int]]] = {}
    with open(log_path, errors="replace") as f:
        for line in f:
            m = re.search(r"\[bench\] timed-window (\S+) (\d+) (\d+)", line)
            if m:
                out.setdefault(m.group(1), []).append((int(m.group(2)), int(m.group(3))))
    return out


def read_rows(run_dir: str, pattern: str) -> List[dict]:
    rows: List[dict] = []
    for path in sorted(glob.glob(os.path.join(run_dir, "**", pattern), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def in_window(row: dict, wins: List[Tuple[int, int]]) -> bool:
    t = int(row["Start_Timestamp"])
    return any(a <= t <= b for a, b in wins)


def short_name(name: str) -> str:
    name = name.strip('"')
    if name.startswith("void "):
        name = name[5:]
    cut = name.find("(wf::")
    return name[:cut] if cut > 0 else name


def cmd_stats(a) -> str:
    wins = windows(a.log).get(a.window, [])
    if not wins:
        raise SystemExit(f"no timed window for {a.window} in {a.log}")
    rows = [r for r in read_rows(a.dir, "*kernel_trace.csv") if in_window(r, wins)]
    if not rows:
        raise SystemExit("no dispatches in the window")
    per: Dict[str, List[float]] = {}
    for r in rows:
        per.setdefault(short_name(r["Kernel_Name"]),
                       []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    steps = sum(1 for r in rows if "prepare_kernel" in r["Kernel_Name"])
    total = sum(sum(v) for v in per.values())
    span = (max(int(r["End_Timestamp"]) for r in rows)
            - min(int(r["Start_Timestamp"]) for r in rows)) / 1e3
    lines = [f"# rocprofv3 kernel statistics -- {a.title}",
             "# command (repo root on the MI355X box):",
             f"#   {a.command}",
             f"# dispatches that start inside the timed window of {a.window} (bench.py",
             f"# --mark-timed): {steps} graph-replayed fixed-block steps, {len(rows)} dispatches;",
             f"# summed kernel time {total / max(steps, 1):.1f} us per step, first start to last end",
             f"# {span / max(steps, 1):.1f} us per step; times in microseconds", "",
             f"{'kernel':<66}{'calls':>7}{'per_step':>9}{'avg_us':>9}{'min_us':>9}{'max_us':>9}"
             f"{'pct':>7}"]
    for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{name[:65]:<66}{len(v):>7}{len(v) / max(steps, 1):>9.1f}"
                     f"{sum(v) / len(v):>9.2f}{min(v):>9.2f}{max(v):>9.2f}"
                     f"{100 * sum(v) / total:>7.2f}")
    return "\n".join(lines) + "\n"


def counter_avg(run_dir: str, log_path: str, window: str, counter: str,
                symbol: str) -> Tuple[float, int, float, float]:
    """(average KiB per dispatch of the kernel in the window, dispatches,
    the largest calibration copy's reading in KiB, the copy's bytes)."""
    wins = windows(log_path)
    kw, cw = wins.get(window, []), wins.get("calibration-copy", [])
    if not kw or not cw:
        raise SystemExit(f"missing windows in {log_path}")
    rows = [r for r in read_rows(run_dir, "*counter_collection.csv")
            if r["Counter_Name"] == counter]
    pat = re.compile(symbol)
    vals = [float(r["Counter_Value"]) for r in rows
            if in_window(r, kw) and pat.search(short_name(r["Kernel_Name"]))]
    cal = [float(r["Counter_Value"]) for r in rows
           if in_window(r, cw) and COPY_KERNEL in r["Kernel_Name"]]
    if not vals or not cal:
        raise SystemExit(f"no {counter} readings for {symbol} or the copy")
    return sum(vals) / len(vals), len(vals), max(cal), 0.0


def cmd_traffic(a) -> str:
    f_avg, n_f, f_cal, _ = counter_avg(a.fetch_dir, a.fetch_log, a.window, "FETCH_SIZE", a.symbol)
    w_avg, n_w, w_cal, _ = counter_avg(a.write_dir, a.write_log, a.window, "WRITE_SIZE", a.symbol)
    copy_kib = a.calib_bytes / 1024.0
    f_scale, w_scale = copy_kib / f_cal, copy_kib / w_cal
    fetch_b = f_avg * f_scale * 1024.0
    write_b = w_avg * w_scale * 1024.0
    total = fetch_b + write_b
    h = kernel_source_hash(a.window)
    text = "\n".join([
        f"# HBM traffic per dispatch -- {a.window}, kernel kind {a.kind}",
        f"# kernels matching {a.symbol!r}: {n_f} dispatches (FETCH_SIZE run), {n_w} (WRITE_SIZE run),",
        "# those starting inside the timed window (bench.py --mark-timed)",
        "# counters: one rocprofv3 run per counter:",
        f"#   {a.command}",
        f"# calibration: the largest device copy of {a.calib_bytes} bytes reads FETCH_SIZE "
        f"{f_cal:.0f} KiB and WRITE_SIZE {w_cal:.0f} KiB: scale {f_scale:.3f} and {w_scale:.3f}",
        "",
        f"FETCH_SIZE avg {f_avg:12.1f} KiB -> {fetch_b / 1e6:10.3f} MB",
        f"WRITE_SIZE avg {w_avg:12.1f} KiB -> {write_b / 1e6:10.3f} MB",
        f"HBM bytes per launch: {total / 1e6:.3f} MB (kernel sources {h})",
        (f"algorithmic bytes per launch: {a.algo_bytes / 1e6:.3f} MB -> traffic / algorithmic "
         f"{total / a.algo_bytes:.3f}") if a.algo_bytes else "",
    ]) + "\n"
    if a.json:
        entries = []
        if os.path.exists(a.json):
            with open(a.json) as f:
                entries = json.load(f)
        entries = [e for e in entries if not (e.get("workload") == a.window
                                              and e.get("kind") == a.kind)]
        entries.append({"workload": a.window, "kind": a.kind, "symbol": a.symbol,
                        "dispatches": n_f, "fetch_kib_avg": f_avg, "write_kib_avg": w_avg,
                        "fetch_scale": f_scale, "write_scale": w_scale,
                        "hbm_bytes_per_launch": total, "algorithmic_bytes": a.algo_bytes or None,
                        "source_hash": h, "command": a.command})
        with open(a.json, "w") as f:
            json.dump(entries, f, indent=1)
            f.write("\n")
    return text


def cmd_mfma(a) -> str:
    """MfmaUtil (MFMA-busy cycles over active cycles times SIMDs) and MFMA
    flops (MfmaFlopsBF16 + MfmaFlopsF16) per dispatch, for the dispatches that
    start inside the timed window, averaged per kernel."""
    wins = windows(a.log).get(a.window, [])
    if not wins:
        raise SystemExit(f"no timed window for {a.window} in {a.log}")
    per: Dict[Tuple[str, str], Dict[str, float]] = {}
    for r in read_rows(a.dir, "*counter_collection.csv"):
        if not in_window(r, wins):
            continue
        c = per.setdefault((short_name(r["Kernel_Name"]), r["Dispatch_Id"]), {})
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    agg: Dict[str, List[float]] = {}
    for (name, _), c in per.items():
        x = agg.setdefault(name, [0, 0.0, 0.0])
        x[0] += 1
        x[1] += c.get("MfmaUtil", 0.0)
        x[2] += c.get("MfmaFlopsBF16", 0.0) + c.get("MfmaFlopsF16", 0.0)
    lines = [f"# rocprofv3 MFMA counters -- {a.title}",
             "# command (repo root on the MI355X box):",
             f"#   {a.command}",
             f"# dispatches that start inside the timed window of {a.window} (bench.py",
             "# --mark-timed); MfmaUtil: MFMA-busy cycles / (active cycles x SIMDs), per",
             "# dispatch; GFLOP: MFMA flops per dispatch (bf16 + fp16)", "",
             f"{'kernel':<66}{'calls':>7}{'mfma_util_%':>13}{'gflop':>11}"]
    for name, (n, u, f) in sorted(agg.items(), key=lambda kv: -kv[1][2]):
        if f <= 0:
            continue
        lines.append(f"{name[:65]:<66}{int(n):>7}{u / n:>13.2f}{f / n / 1e9:>11.3f}")
    return "\n".join(lines) + "\n"


def main(argv: Optional[List[str]] = None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--dir", required=True)
    s.add_argument("--log", required=True)
    s.add_argument("--window", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out")
    mf = sub.add_parser("mfma")
    for k in ("dir", "log", "window", "title", "command"):
        mf.add_argument("--" + k, required=True)
    mf.add_argument("--out")
    t = sub.add_parser("traffic")
    for k in ("fetch-dir", "fetch-log", "write-dir", "write-log", "window", "kind", "symbol",
              "command"):
        t.add_argument("--" + k, required=True)
    t.add_argument("--calib-bytes", type=float, default=256.0 * 2 ** 20)
    t.add_argument("--algo-bytes", type=float, default=0.0)
    t.add_argument("--out")
    t.add_argument("--json")
    a = ap.parse_args(argv)
    text = {"stats": cmd_stats, "mfma": cmd_mfma, "traffic": cmd_traffic}[a.cmd](a)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
