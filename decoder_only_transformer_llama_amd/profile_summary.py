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

* ``counters``: per kernel, the SQ/GRBM counters of one or more ``--pmc``
  runs with what follows from them: the fraction of SIMD cycles the matrix
  cores were busy (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE per XCD times
  the SIMD count), the clock the kernel ran at (GUI-active cycles per XCD over
  the dispatch's duration), non-matrix VALU instructions per MFMA, LDS bank
  conflict cycles per LDS instruction; and, with ``--bytes`` runs
  (FETCH_SIZE / WRITE_SIZE), HBM GB/s per kernel.

Usage:
  python -m decoder_only_transformer_llama_amd.profile_summary stats DIR OUT.txt --command "..."
  python -m decoder_only_transformer_llama_amd.profile_summary counters OUT.txt --pmc DIR [DIR ...] \
      [--fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes N] --command "..."
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


def _bench_line(path: str) -> Optional[dict]:
    """The JSON line bench.py printed (the last line of the log that parses as an object)."""
    import json
    found = None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                try:
                    found = json.loads(line)
                except ValueError:
                    pass
    return found


def write_stats(d: str, out: str, command: str, top: int, bench_log: Optional[str] = None,
                roofline: Optional[List[str]] = None) -> None:
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
    # roofline objects of the bench line printed by this same run, recomputed
    # from the trace median of the kernel they name: (path in the line, kernel)
    line = _bench_line(bench_log) if bench_log else None
    if line is not None:
        lines += ["", "bench.py line of this run (ms_per_step %s):" % line.get("ms_per_step")]
        for spec in roofline or []:
            path, kern = spec.split("=", 1)
            obj = line
            for key in path.split("."):
                obj = obj.get(key, {}) if isinstance(obj, dict) else {}
            # KERNEL may be several '+'-joined substrings (one launch each, all
            # timed together by the line): their trace medians add up
            parts = kern.split("+")
            m = [[v for k, v in med.items() if part in k] for part in parts]
            if not obj or not all(m):
                continue
            t_ns = sum(x[0] for x in m)
            per = obj.get("flops_per_launch") or obj.get("bytes_per_launch")
            scale = 1e-3 if obj.get("unit") == "TFLOP/s" else 1.0   # per ns -> TFLOP/s (1e-3) or GB/s (1)
            rec = per / t_ns * scale
            lines += [f"  {path}: {obj.get('kernel')}",
                      f"    line: achieved {obj.get('achieved')} {obj.get('unit')}, frac {obj.get('frac')}, "
                      f"traffic {obj.get('traffic')}",
                      f"    trace median of {' + '.join(repr(p) for p in parts)}: {t_ns / 1e3:.2f} us -> "
                      f"{rec:.1f} {obj.get('unit')}, frac {rec / obj.get('peak'):.4f}"]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_traffic(a) -> None:
    # one or more kernels (--kernel repeated: the launches of one step, e.g. a
    # GEMM split into two column ranges); their per-dispatch means add up
    cf, ncf = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cw, ncw = counter_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    f_fetch = cf * 1024.0 / a.copy_bytes
    f_write = cw * 1024.0 / a.copy_bytes
    traffic, per_kernel = 0.0, []
    for k in a.kernel:
        fetch, nf = counter_per_dispatch(a.fetch, "FETCH_SIZE", k)
        write, nw = counter_per_dispatch(a.write, "WRITE_SIZE", k)
        traffic += fetch * 1024.0 / f_fetch + write * 1024.0 / f_write
        per_kernel += [f"{k}:",
                       f"  FETCH_SIZE per dispatch: {fetch:.1f} KiB (mean of {nf} dispatches)",
                       f"  WRITE_SIZE per dispatch: {write:.1f} KiB (mean of {nw} dispatches)"]
    lines = [
        "# HBM traffic per launch from rocprofv3 counters",
        "",
        f"kernel: {' + '.join(a.kernel)}",
        "commands:",
    ] + ["  " + c for c in a.command] + [""] + per_kernel + [
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


def _agent(d: str) -> Dict[str, float]:
    """Num_Xcc, Simd_Count and Max_Engine_Clk_Fcompute of the GPU agent of a run."""
    for f in _find(d, "agent_info.csv"):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r.get("Agent_Type") == "GPU":
                    return {k: float(r[k]) for k in ("Num_Xcc", "Simd_Count", "Max_Engine_Clk_Fcompute")}
    raise SystemExit(f"no GPU agent_info.csv under {d}")


def per_kernel_counters(dirs: List[str]) -> Dict[str, Dict[str, float]]:
    """{kernel: {counter: mean per dispatch, '_n': dispatches, '_dur_ns': median duration}}"""
    out: Dict[str, Dict[str, float]] = {}
    for d in dirs:
        per: Dict[Tuple[str, str], Dict[str, float]] = {}
        durs: Dict[Tuple[str, str], int] = {}
        for f in _find(d, "counter_collection.csv"):
            with open(f, newline="") as fh:
                for r in csv.DictReader(fh):
                    key = (r["Kernel_Name"], f + ":" + r["Dispatch_Id"])
                    c = per.setdefault(key, {})
                    c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                    durs[key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        by_k: Dict[str, List[Tuple[Dict[str, float], int]]] = {}
        for (k, disp), c in per.items():
            by_k.setdefault(k, []).append((c, durs[(k, disp)]))
        for k, lst in by_k.items():
            o = out.setdefault(k, {})
            for name in lst[0][0]:
                o[name] = sum(c.get(name, 0.0) for c, _ in lst) / len(lst)
            o["_n"] = len(lst)
            ds = sorted(t for _, t in lst)
            o.setdefault("_dur_ns", float(ds[len(ds) // 2]))
    return out


def write_counters(a) -> None:
    ag = _agent(a.pmc[0])
    xcc, simds, mhz = ag["Num_Xcc"], ag["Simd_Count"], ag["Max_Engine_Clk_Fcompute"]
    kc = per_kernel_counters(a.pmc)
    f_fetch = f_write = None
    if a.fetch:
        cf, _ = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
        cw, _ = counter_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)
        f_fetch, f_write = cf * 1024.0 / a.copy_bytes, cw * 1024.0 / a.copy_bytes
        for k, v in per_kernel_counters([a.fetch, a.write]).items():
            o = kc.setdefault(k, {"_n": v["_n"], "_dur_ns": v["_dur_ns"]})
            for name in ("FETCH_SIZE", "WRITE_SIZE"):
                if name in v:
                    o[name] = v[name]
            o["_bytes_dur_ns"] = v["_dur_ns"]
    rows = []
    for k, c in kc.items():
        if not any(s in k for s in a.kernel) and a.kernel:
            continue
        rows.append((k, c))
    rows.sort(key=lambda kv: -kv[1].get("SQ_VALU_MFMA_BUSY_CYCLES", kv[1].get("FETCH_SIZE", 0.0)))
    lines = ["# rocprofv3 counters per kernel (means per dispatch)", "", "commands:"] + ["  " + c for c in a.command]
    lines += ["", f"GPU: {int(xcc)} XCDs, {int(simds)} SIMDs, peak engine clock {mhz:.0f} MHz", "",
              "mfma_busy: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs * SIMDs), at the clock the kernel ran",
              "clock: GRBM_GUI_ACTIVE / XCDs / dispatch duration under counters ('-' where that exceeds the peak",
              "  clock: for short kernels the GUI-active count includes time outside the dispatch)",
              "peak_frac = mfma_busy * clock / peak clock: the fraction of the 2.5 PFLOP/s dense fp16/bf16 peak",
              "valu/mfma: (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA (SQ_INSTS_VALU counts MFMAs too)",
              "lds_conf: SQ_LDS_BANK_CONFLICT cycles per SQ_INSTS_LDS instruction"]
    if f_fetch:
        lines += [f"HBM bytes: FETCH_SIZE / {f_fetch:.4f} + WRITE_SIZE / {f_write:.4f} (factors from a {a.copy_kernel} "
                  f"copy of {a.copy_bytes} bytes); GB/s over the dispatch's duration in the byte-counter runs"]
    lines += ["", f"{'n':>4} {'dur us':>9} {'mfma':>10} {'busy':>6} {'clk GHz':>7} {'peak_fr':>7} {'valu/mfma':>9} "
              f"{'lds_conf':>8} {'MB':>9} {'GB/s':>7}  kernel"]
    for k, c in rows:
        n = int(c["_n"])
        dur = c["_dur_ns"]
        gui = c.get("GRBM_GUI_ACTIVE")
        mf = c.get("SQ_INSTS_MFMA")
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
        cyc = gui / xcc if gui else None
        fb = busy / (cyc * simds) if busy is not None and cyc else None
        clk = cyc / dur if cyc and dur else None
        if clk is not None and clk > 1.05 * mhz / 1e3:
            clk = None   # GUI-active cycles outside the dispatch dominate a short kernel: no clock estimate
        pf = fb * clk / (mhz / 1e3) if fb is not None and clk else None
        vpm = (c["SQ_INSTS_VALU"] - mf) / mf if mf and "SQ_INSTS_VALU" in c else None
        lc = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_INSTS_LDS"] if c.get("SQ_INSTS_LDS") and "SQ_LDS_BANK_CONFLICT" in c else None
        mb = gbs = None
        if f_fetch and "FETCH_SIZE" in c and "WRITE_SIZE" in c:
            byt = c["FETCH_SIZE"] * 1024.0 / f_fetch + c["WRITE_SIZE"] * 1024.0 / f_write
            mb = byt / 1e6
            gbs = byt / c.get("_bytes_dur_ns", dur)
        fmt = lambda v, w, p: f"{v:{w}.{p}f}" if v is not None else f"{'-':>{w}}"
        lines.append(f"{n:4d} {dur / 1e3:9.2f} {fmt(mf, 10, 0)} {fmt(fb, 6, 3)} {fmt(clk, 7, 3)} {fmt(pf, 7, 3)} "
                     f"{fmt(vpm, 9, 2)} {fmt(lc, 8, 3)} {fmt(mb, 9, 2)} {fmt(gbs, 7, 0)}  {short_name(k)}")
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
    s.add_argument("--bench-log", help="output of the profiled bench.py run (its JSON line)")
    s.add_argument("--roofline", action="append", default=[],
                   help="PATH=KERNEL: a roofline object of the line (e.g. roofline or decode.roofline) and a "
                        "substring of the kernel it times ('+'-joined substrings: launches timed together)")
    t = sub.add_parser("traffic")
    t.add_argument("out")
    t.add_argument("--kernel", action="append", required=True,
                   help="substring of the kernel's name; repeat for the launches of one step (summed)")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--sources", nargs="+", required=True)
    t.add_argument("--command", action="append", required=True)
    c = sub.add_parser("counters")
    c.add_argument("out")
    c.add_argument("--pmc", nargs="+", required=True)
    c.add_argument("--kernel", action="append", default=[], help="keep kernels whose name contains this")
    c.add_argument("--fetch")
    c.add_argument("--write")
    c.add_argument("--copy-fetch")
    c.add_argument("--copy-write")
    c.add_argument("--copy-kernel", default="copy")
    c.add_argument("--copy-bytes", type=int)
    c.add_argument("--command", action="append", required=True)
    a = ap.parse_args()
    if a.cmd == "stats":
        write_stats(a.dir, a.out, a.command, a.top, a.bench_log, a.roofline)
    elif a.cmd == "counters":
        write_counters(a)
    else:
        write_traffic(a)


if __name__ == "__main__":
    main()
