"""Summaries of rocprofv3 output for the kernels of libpariskv.so.

Two kinds of summary are written as short text files:

* kernel statistics (``--kernel-trace --stats``): calls and average / min / max
  duration per kernel;
* HBM traffic per launch of one kernel from two counter runs, one collecting
  ``FETCH_SIZE`` and one ``WRITE_SIZE`` (KiB per dispatch).  Each counter is
  scaled by what it reads for a plain 16-byte-per-lane streaming copy of known
  size (``pk_calibration_copy``), so that the request-size accounting of the
  counter cancels out.  The file records a digest of the kernel sources; a
  traffic figure whose digest no longer matches the sources is stale and
  ``load_traffic`` returns None for it.

    python -m kv_cache_top_amd.profiling stats  KERNEL_STATS_CSV OUT --command "..."
    python -m kv_cache_top_amd.profiling traffic FETCH_CSV WRITE_CSV OUT --kernel collide
            --workload batched128k --alg-bytes N --command-fetch "..." --command-write "..."
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
SOURCES = ("csrc/pk_kernels.hpp", "csrc/pk_api.hip")
CALIBRATION_KERNEL = "copy16_kernel"


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(full: str) -> str:
    """'void pk::collide_kernel<4>(...)' -> 'collide_kernel<4>'."""
    name = full.split("(")[0].replace("void ", "").strip()
    return name.split("::")[-1] if name.startswith("pk::") else name


# kernels that pk_timing brackets under another kernel's name
KEY_ALIASES = {"select_sub": "select", "append_qprep": "qprep"}


def kernel_key(full: str) -> str:
    """'void pk::collide_kernel<4>(...)' -> 'collide' (the names pk_timing uses)."""
    s = short_name(full)
    k = s.split("_kernel")[0] if "_kernel" in s else s
    return KEY_ALIASES.get(k, k)


def _per_kernel(counter_csv: str, counter: str) -> dict:
    vals = defaultdict(list)
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def summarize_stats(stats_csv: str, out: str, command: str) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = ["# rocprofv3 kernel statistics", "", "Command:", "", "    " + command, "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    lines += ["", f"kernel source digest: {kernel_source_digest()}", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines))


def summarize_traffic(fetch_csv: str, write_csv: str, out: str, kernel: str, workload: str, alg_bytes: int,
                      command_fetch: str, command_write: str, calibration_bytes: int = 1 << 30) -> dict:
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")

    def pick(vals, key):
        # the instantiation with the most dispatches (the timed one; a run may
        # also make a few other calls, e.g. a retrieval without attention)
        hits = {k: v for k, v in vals.items() if kernel_key(k) == key}
        if not hits:
            raise SystemExit(f"no kernel named {key!r}")
        name, v = max(hits.items(), key=lambda kv: len(kv[1]))
        return short_name(name), v

    kname, fk = pick(fetch, kernel)
    _, wk = pick(write, kernel)
    _, fc = pick(fetch, CALIBRATION_KERNEL.split("_kernel")[0])
    _, wc = pick(write, CALIBRATION_KERNEL.split("_kernel")[0])
    fetch_kib = sum(fk) / len(fk)
    write_kib = sum(wk) / len(wk)
    cal_fetch_kib = max(fc)          # the calibration copy moves calibration_bytes each way
    cal_write_kib = max(wc)
    f_fac = calibration_bytes / (cal_fetch_kib * 1024.0)
    w_fac = calibration_bytes / (cal_write_kib * 1024.0)
    read_b = fetch_kib * 1024.0 * f_fac
    write_b = write_kib * 1024.0 * w_fac
    res = {
        "kernel": kernel, "kernel_symbol": kname, "workload": workload, "dispatches": len(fk),
        "fetch_kib_per_dispatch": round(fetch_kib, 1), "write_kib_per_dispatch": round(write_kib, 1),
        "calibration_copy_bytes": calibration_bytes,
        "calibration_fetch_kib": round(cal_fetch_kib, 1), "calibration_write_kib": round(cal_write_kib, 1),
        "fetch_scale": round(f_fac, 4), "write_scale": round(w_fac, 4),
        "hbm_read_bytes_per_launch": int(read_b), "hbm_write_bytes_per_launch": int(write_b),
        "hbm_bytes_per_launch": int(read_b + write_b),
        "algorithmic_bytes_per_launch": int(alg_bytes),
        "traffic_over_algorithmic": round((read_b + write_b) / alg_bytes, 3) if alg_bytes else None,
        "kernel_source_digest": kernel_source_digest(),
    }
    lines = [f"# HBM traffic of {kernel} on {workload} (rocprofv3 counters)", "",
             "Fetch command:", "", "    " + command_fetch, "", "Write command:", "", "    " + command_write, ""]
    lines += [f"{k}: {v}" for k, v in res.items()]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return res


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload`, or None (no summary, or stale)."""
    path = os.path.join(PROFILES, f"pmc_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ": " in line and not line.startswith(("#", " ")):
            k, v = line.rstrip("\n").split(": ", 1)
            kv[k] = v
    if kv.get("kernel_source_digest") != kernel_source_digest():
        return None
    return int(kv["hbm_bytes_per_launch"])


def load_trace_avg_us(kernel: str, workload: str):
    """Average rocprofv3 trace duration (us) of `kernel` (the pk_timing name) on
    `workload` from profiles/kernels_<workload>.md, or None (no summary, no
    such kernel, or stale: the summary's source digest differs)."""
    path = os.path.join(PROFILES, f"kernels_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if f"kernel source digest: {kernel_source_digest()}" not in text:
        return None
    hits = []
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 3 and "_kernel" in cells[0]:
            if kernel_key(cells[0]) == kernel:
                hits.append((int(cells[1]), float(cells[2])))
    if not hits:
        return None
    calls = sum(c for c, _ in hits)
    return round(sum(c * us for c, us in hits) / calls, 3)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("out")
    a.add_argument("--command", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("out")
    b.add_argument("--kernel", required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--alg-bytes", type=int, required=True)
    b.add_argument("--command-fetch", required=True)
    b.add_argument("--command-write", required=True)
    args = ap.parse_args()
    if args.cmd == "stats":
        summarize_stats(args.csv, args.out, args.command)
    else:
        print(summarize_traffic(args.fetch_csv, args.write_csv, args.out, args.kernel, args.workload,
                                args.alg_bytes, args.command_fetch, args.command_write))


if __name__ == "__main__":
    main()
