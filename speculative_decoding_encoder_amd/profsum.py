"""Summaries of rocprofv3 output for the verify path (text for profiles/).

  python -m speculative_decoding_encoder_amd.profsum stats DIR TITLE CMD
      per-kernel statistics of a --kernel-trace --stats run (run_kernel_stats.csv)
  python -m speculative_decoding_encoder_amd.profsum traffic FETCH_DIR WRITE_DIR WORKLOAD KIND
          SYMBOL COPY_BYTES OUT_TXT CMD
      HBM bytes per dispatch of the kernels whose name starts with SYMBOL,
      from a FETCH_SIZE run and a WRITE_SIZE run of the same command (KiB per
      dispatch), each scaled by what the counter reads for the largest buffer
      copy in the run (COPY_BYTES read and written); appends the figure to
      profiles/hbm_traffic.json, keyed by workload, kernel kind and a hash of
      the workload's kernel sources, and writes a text summary to OUT_TXT.
  python -m speculative_decoding_encoder_amd.profsum mfma DIR TITLE CMD
      per-kernel MFMA utilisation (MfmaUtil: MFMA-busy cycles over active
      cycles times SIMDs) and MFMA flops per dispatch (MfmaFlopsBF16 +
      MfmaFlopsF16) of a --pmc MfmaUtil MfmaFlopsBF16 MfmaFlopsF16 run.
"""
from __future__ import annotations

import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _short(name: str, n: int = 64) -> str:
    name = name.replace("void ", "").replace("(wf::GemmArgs)", "")
    return name if len(name) <= n else name[: n - 1] + "~"


def stats(d: str, title: str, cmd: str) -> str:
    rows = list(csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv"))))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# rocprofv3 kernel statistics -- {title}",
           "# command (repo root on the MI355X box):", f"#   {cmd}",
           "# all dispatches of the run (set-up, warm-up, graph-replayed timed steps and the",
           "# event-timed pass); times in microseconds", "",
           f"{'kernel':66s} {'calls':>7s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for r in rows[:40]:
        out.append(f"{_short(r['Name'], 66):66s} {int(r['Calls']):7d} "
                   f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                   f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}")
    return "\n".join(out) + "\n"


def _per_dispatch(d: str, counter: str):
    """{(kernel name, dispatch id): (grid size, counter value summed over agents)}"""
    vals = {}
    for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        g, v = vals.get(key, (int(r["Grid_Size"]), 0.0))
        vals[key] = (g, v + float(r["Counter_Value"]))
    return vals


def traffic(fdir, wdir, workload, kind, symbol, copy_bytes, out_txt, cmd):
    fetch = _per_dispatch(fdir, "FETCH_SIZE")
    write = _per_dispatch(wdir, "WRITE_SIZE")

    def pick(vals, prefix):
        # the dispatches of the most frequent grid size (the timed passes;
        # set-up launches such as prefill blocks run other grids)
        sel = [(g, v) for (name, _), (g, v) in vals.items()
               if name.replace("void ", "").startswith(prefix)]
        if not sel:
            return []
        grids = [g for g, _ in sel]
        mode = max(set(grids), key=grids.count)
        return [v for g, v in sel if g == mode]

    def copy_kib(vals):
        c = [v for (name, _), (g, v) in vals.items() if "copyBuffer" in name]
        return max(c) if c else None

    cf, cw = copy_kib(fetch), copy_kib(write)
    kf, kw = pick(fetch, symbol), pick(write, symbol)
    if not kf or not kw or not cf or not cw:
        raise SystemExit(f"missing dispatches: kernel {len(kf)}/{len(kw)}, copy {cf}/{cw}")
    sf = copy_bytes / (cf * 1024.0)
    sw = copy_bytes / (cw * 1024.0)
    f_b = sum(kf) / len(kf) * 1024.0 * sf
    w_b = sum(kw) / len(kw) * 1024.0 * sw
    sys.path.insert(0, ROOT)
    from bench import kernel_source_hash
    h = kernel_source_hash(workload)
    ent = {"workload": workload, "kind": kind, "symbol": symbol, "dispatches": len(kf),
           "fetch_kib_avg": sum(kf) / len(kf), "write_kib_avg": sum(kw) / len(kw),
           "fetch_scale": sf, "write_scale": sw, "hbm_bytes_per_launch": f_b + w_b,
           "source_hash": h, "command": cmd}
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    entries = []
    if os.path.exists(path):
        entries = [e for e in json.load(open(path))
                   if not (e.get("workload") == workload and e.get("kind") == kind)]
    entries.append(ent)
    with open(path, "w") as f:
        json.dump(entries, f, indent=1)
    txt = [f"# HBM traffic per dispatch -- {workload}, kernel kind {kind}",
           f"# kernels: {symbol}* ({len(kf)} dispatches)",
           "# counters: rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE, one run each:",
           f"#   {cmd}",
           f"# calibration: the largest buffer copy of the run, {copy_bytes} bytes read and",
           f"# written, reads FETCH_SIZE {cf:.0f} KiB and WRITE_SIZE {cw:.0f} KiB: scale "
           f"{sf:.3f} and {sw:.3f}", "",
           f"FETCH_SIZE avg {sum(kf) / len(kf):12.1f} KiB -> {f_b / 1e6:10.3f} MB",
           f"WRITE_SIZE avg {sum(kw) / len(kw):12.1f} KiB -> {w_b / 1e6:10.3f} MB",
           f"HBM bytes per launch: {(f_b + w_b) / 1e6:.3f} MB (kernel sources {h})"]
    with open(out_txt, "w") as f:
        f.write("\n".join(txt) + "\n")
    return ent


def mfma(d: str, title: str, cmd: str) -> str:
    per = {}
    for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        per.setdefault(key, {})[r["Counter_Name"]] = \
            per.get(key, {}).get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    agg = {}
    for (name, _), c in per.items():
        a = agg.setdefault(name, [0, 0.0, 0.0])
        a[0] += 1
        a[1] += c.get("MfmaUtil", 0.0)
        a[2] += c.get("MfmaFlopsBF16", 0.0) + c.get("MfmaFlopsF16", 0.0)
    rows = sorted(agg.items(), key=lambda kv: -kv[1][2])
    out = [f"# rocprofv3 MFMA counters -- {title}", "# command (repo root on the MI355X box):",
           f"#   {cmd}", "# MfmaUtil: MFMA-busy cycles / (active cycles x SIMDs), per dispatch;",
           "# GFLOP: MFMA flops per dispatch (bf16 + fp16 MOPS x 512)", "",
           f"{'kernel':66s} {'calls':>7s} {'mfma_util_%':>11s} {'gflop':>10s}"]
    for name, (n, u, f) in rows:
        if f <= 0:
            continue
        out.append(f"{_short(name, 66):66s} {n:7d} {u / n:11.2f} {f / n / 1e9:10.3f}")
    return "\n".join(out) + "\n"


def main(argv):
    if argv and argv[0] == "stats":
        sys.stdout.write(stats(argv[1], argv[2], " ".join(argv[3:])))
    elif argv and argv[0] == "mfma":
        sys.stdout.write(mfma(argv[1], argv[2], " ".join(argv[3:])))
    elif argv and argv[0] == "traffic":
        ent = traffic(argv[1], argv[2], argv[3], argv[4], argv[5], float(argv[6]), argv[7],
                      " ".join(argv[8:]))
        print(json.dumps(ent))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
