"""Summaries of rocprofv3 CSV output as short text files.

Two summaries:

* ``stats``: the kernel table of a ``rocprofv3 --kernel-trace --stats
  --output-format csv`` run (calls, total and average duration per kernel);
* ``traffic``: HBM bytes per launch of one kernel from two ``--pmc`` runs
  (``FETCH_SIZE``, then ``WRITE_SIZE``; both count KiB per dispatch),
  each divided by the factor the same counter shows for a plain device copy of
  known size, so that ``traffic = FETCH/f_fetch + WRITE/f_write`` in bytes.
  The summary records the SHA-256 of the kernel's source files; bench.py
  reports the figure only while those sources are unchanged.

Usage:
  python -m decoder_only_transformer_llama_amd.profile_summary stats DIR OUT.txt --command "..."
  python -m decoder_only_transformer_llama_amd.profile_summary traffic --kernel SUBSTR \\
      --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes N \\
      --sources a.hip b.h --command "..." OUT.txt
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
from typing import Dict, List, Optional, Tuple

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _find(d: str, suffix: str) -> List[str]:
    return sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))


def short_name(name: str, width: int = 90) -> str:
    name = name.strip()
    if name.endswith(")"):                                # drop the trailing argument list
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                name = name[:i]
                break
    if name.startswith("void "):
        name = name[5:]
    return name if len(name) <= width else name[: width - 3] + "..."


def sources_sha256(paths: List[str]) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(p.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()


def stats_table(d: str) -> List[Tuple[str, int, float, float, float]]:
    files = _find(d, "kernel_stats.csv")
    if not files:
        raise SystemExit(f"no *kernel_stats.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                rows.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]), float(r["AverageNs"]),
                             float(r["Percentage"])))
    rows.sort(key=lambda r: -r[2])
    return rows


def counter_per_dispatch(d: str, counter: str, kernel: str) -> Tuple[float, int]:
    """Mean value of `counter` over dispatches whose name contains `kernel`."""
    files = _find(d, "counter_collection.csv")
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    vals: Dict[str, float] = {}
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter or kernel not in r["Kernel_Name"]:
                    continue
                key = f + ":" + r["Dispatch_Id"]
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel!r} under {d}")
    return sum(vals.values()) / len(vals), len(vals)


def trace_medians(d: str) -> Dict[str, float]:
    """Median duration (ns) per kernel name from the run's kernel trace."""
    durs: Dict[str, List[int]] = {}
    for f in _find(d, "kernel_trace.csv"):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                durs.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = {}
    for k, v in durs.items():
        v.sort()
        n = len(v)
        out[k] = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return out


def write_stats(d: str, out: str, command: str, top: int) -> None:
    rows = stats_table(d)
    med = trace_medians(d)
    total = sum(r[2] for r in rows)
    lines = ["# rocprofv3 kernel statistics", "", "command:", "  " + command, "",
             "avg: rocprofv3's mean over every dispatch; median: from the kernel trace of the same run",
             "(calls right after an idle gap, while the clock ramps up, pull the mean above the median)", "",
             f"{'avg us':>10} {'median us':>10} {'calls':>6} {'total ms':>9} {'%':>6}  kernel"]
    for name, calls, tot, avg, pct in rows[:top]:
        m = med.get(name)
        ms = f"{m / 1e3:10.2f}" if m is not None else f"{'-':>10}"
        lines.append(f"{avg / 1e3:10.2f} {ms} {calls:6d} {tot / 1e6:9.3f} {pct:6.2f}  {short_name(name)}")
    lines += ["", f"all kernels: {total / 1e6:.3f} ms over {sum(r[1] for r in rows)} dispatches"]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_traffic(a) -> None:
    fetch, nf = counter_per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    write, nw = counter_per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    cf, ncf = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cw, ncw = counter_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    f_fetch = cf * 1024.0 / a.copy_bytes
    f_write = cw * 1024.0 / a.copy_bytes
    traffic = fetch * 1024.0 / f_fetch + write * 1024.0 / f_write
    lines = [
        "# HBM traffic per launch from rocprofv3 counters",
        "",
        f"kernel: {a.kernel}",
        "commands:",
    ] + ["  " + c for c in a.command] + [
        "",
        f"FETCH_SIZE per dispatch: {fetch:.1f} KiB (mean of {nf} dispatches)",
        f"WRITE_SIZE per dispatch: {write:.1f} KiB (mean of {nw} dispatches)",
        f"copy calibration ({a.copy_kernel}, {a.copy_bytes} bytes read and written per dispatch):",
        f"  FETCH_SIZE {cf:.1f} KiB over {ncf} dispatches -> factor {f_fetch:.4f}",
        f"  WRITE_SIZE {cw:.1f} KiB over {ncw} dispatches -> factor {f_write:.4f}",
        "",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        f"sources: {' '.join(a.sources)}",
        f"source_sha256: {sources_sha256(a.sources)}",
    ]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def stored_traffic(path: str) -> Optional[float]:
    """traffic_bytes_per_launch from a summary written by `traffic`, or None
    when the file is missing or the kernel's sources changed since."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    try:
        srcs = kv["sources"].split()
        if sources_sha256(srcs) != kv["source_sha256"]:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError, OSError):
        return None


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    s.add_argument("--top", type=int, default=25)
    t = sub.add_parser("traffic")
    t.add_argument("out")
    t.add_argument("--kernel", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--sources", nargs="+", required=True)
    t.add_argument("--command", action="append", required=True)
    a = ap.parse_args()
    if a.cmd == "stats":
        write_stats(a.dir, a.out, a.command, a.top)
    else:
        write_traffic(a)


if __name__ == "__main__":
    main()
