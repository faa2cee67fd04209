"""Turns rocprofv3 CSV output into the short text summaries kept beside the library.

Two reports:

  stats    per (kernel, grid) launch count and duration (avg/min/max, microseconds) from a
           ``--kernel-trace --output-format csv`` run, so that launches of one kernel on
           different workloads are not averaged together.
  traffic  HBM bytes per dispatch from two ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs.
           Each counter is scaled by what it reads for a plain device copy of known size in
           the same run (the largest ``__amd_rocclr_copyBuffer`` dispatch), so the factor
           is measured, not assumed.

  counters per-dispatch means of the counters of one ``--pmc`` run for selected kernels, with
           the clock (GRBM_GUI_ACTIVE counts every XCD's cycles) and, when
           SQ_VALU_MFMA_BUSY_CYCLES is among them, the fraction of the kernel's cycles the
           matrix cores of an average SIMD were busy (the counter sums all SIMDs' busy cycles).

The traffic report ends with machine-readable lines (``key: value``) that bench.py reads; the
``sources_sha256`` line ties the counters to the kernel sources they were taken with.

    python -m value_only_kv_amd.profile_summary stats TRACE_CSV --cmd "..." -o OUT.md
    python -m value_only_kv_amd.profile_summary traffic FETCH_CSV WRITE_CSV --copy-bytes N \
        --select NAME:GRID [--select NAME:GRID ...] --algorithmic-bytes B --cmd "..." -o OUT.md
    python -m value_only_kv_amd.profile_summary counters PMC_CSV --select NAME:GRID [...] \
        --cmd "..." -o OUT.md
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os

PKG = os.path.dirname(os.path.abspath(__file__))

# Sources whose change invalidates stored decode counters.
DECODE_SOURCES = ("csrc/k_decode_mfma.hip", "csrc/k_decode_generic.hip", "csrc/gva_api.hip",
                  "csrc/gva_host.cpp", "csrc/gva_internal.h", "csrc/gva_device.h")


def sources_sha256(paths=DECODE_SOURCES) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(PKG, p), "rb") as f:
            h.update(p.encode() + b"\0" + f.read())
    return h.hexdigest()


def _short(name: str) -> str:
    n = name.replace("void ", "").replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(n):               # drop the parameter list (the first "(" outside <>)
        depth += (ch == "<") - (ch == ">")
        if ch == "(" and depth == 0:
            n = n[:i]
            break
    if n.startswith(("at::", "__amd")):
        n = "(input generation) " + n.split("<")[0]
    return n


def stats(trace_csv: str, cmd: str, note: str = "", splits=(), only=()) -> str:
    """splits: "NAME:US" entries; the launches of a kernel whose name contains NAME are reported
    in two rows, below and at or above US microseconds (one grid run on two workload sizes).
    only: report just the kernels whose names contain one of these strings."""
    cut = {}
    for sp in splits:
        name, us = sp.rsplit(":", 1)
        cut[name] = float(us) * 1e3
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        if only and not any(o in r["Kernel_Name"] for o in only):
            continue
        grid = (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]))
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        name = _short(r["Kernel_Name"])
        for sub, ns in cut.items():
            if sub in r["Kernel_Name"]:
                name += f" (< {ns / 1e3:g} us)" if d < ns else f" (>= {ns / 1e3:g} us)"
        agg[(name, grid, wg)].append(d)
    lines = ["# rocprofv3 kernel trace summary", "", "Command:", "", "```", cmd, "```", "",
             "Per kernel and launch grid (grid in threads x, y, z; work-group size); durations "
             "in microseconds.", "", *([note, ""] if note else []),
             "| kernel | grid | wg | calls | avg us | median us | min us | max us | total ms |",
             "|---|---|---|---|---|---|---|---|---|"]
    for (k, g, wg), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        srt = sorted(v)
        n = len(srt)
        med = srt[n // 2] if n % 2 else (srt[n // 2 - 1] + srt[n // 2]) / 2
        lines.append(f"| `{k}` | {g[0]}x{g[1]}x{g[2]} | {wg} | {n} | "
                     f"{sum(v) / n / 1e3:.2f} | {med / 1e3:.2f} | {min(v) / 1e3:.2f} | "
                     f"{max(v) / 1e3:.2f} | {sum(v) / 1e6:.3f} |")
    return "\n".join(lines) + "\n"


def _counter_rows(path: str):
    out = []
    for r in csv.DictReader(open(path)):
        out.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
    return out


def traffic(fetch_csv: str, write_csv: str, copy_bytes: int, selects, algorithmic: int,
            cmd: str, note: str = "") -> str:
    fetch, write = _counter_rows(fetch_csv), _counter_rows(write_csv)

    def copy_kib(rows):
        vals = [v for n, _, v in rows if "copyBuffer" in n]
        if not vals:
            raise SystemExit("no device copy dispatch in the counter run (use --copy-calibration)")
        return max(vals)

    f_scale = copy_bytes / (copy_kib(fetch) * 1024.0)
    w_scale = copy_bytes / (copy_kib(write) * 1024.0)
    lines = ["# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Commands (one counter per run):", "", "```", cmd, "```", "",
             *([note, ""] if note else []),
             f"Calibration: a plain device copy of {copy_bytes} bytes reads FETCH_SIZE "
             f"{copy_kib(fetch):.0f} KiB and WRITE_SIZE {copy_kib(write):.0f} KiB, so the "
             f"counters are scaled by {f_scale:.4f} (fetch) and {w_scale:.4f} (write).", "",
             "| kernel | grid (threads) | dispatches | FETCH KiB (raw avg) | WRITE KiB (raw avg) "
             "| HBM read bytes | HBM write bytes |", "|---|---|---|---|---|---|---|"]
    total = 0.0
    for sel in selects:
        name, grid = sel.rsplit(":", 1)
        grid = int(grid)
        fv = [v for n, g, v in fetch if name in n and g == grid]
        wv = [v for n, g, v in write if name in n and g == grid]
        if not fv or not wv:
            raise SystemExit(f"no dispatch of {name} with grid {grid}")
        fa, wa = sum(fv) / len(fv), sum(wv) / len(wv)
        rb, wb = fa * 1024 * f_scale, wa * 1024 * w_scale
        total += rb + wb
        lines.append(f"| `{name}` | {grid} | {len(fv)} | {fa:.0f} | {wa:.0f} | {rb:.4g} | "
                     f"{wb:.4g} |")
    lines += ["", f"Algorithmic bytes per call: {algorithmic}; measured HBM traffic per call: "
              f"{total:.6g} bytes ({total / algorithmic:.4f}x).", "",
              f"traffic_bytes_per_call: {int(round(total))}",
              f"algorithmic_bytes_per_call: {algorithmic}",
              f"sources_sha256: {sources_sha256()}"]
    return "\n".join(lines) + "\n"


MI355X_XCDS = 8
MI355X_SIMDS = 256 * 4


def counters(pmc_csv: str, selects, cmd: str, note: str = "") -> str:
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    durs = collections.defaultdict(dict)
    names = []
    for r in csv.DictReader(open(pmc_csv)):
        key = (r["Kernel_Name"], int(r["Grid_Size"]))
        vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
        durs[key][r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if r["Counter_Name"] not in names:
            names.append(r["Counter_Name"])
    sized = ("TCC_EA0_RDREQ_128B", "TCC_EA0_RDREQ_64B", "TCC_EA0_RDREQ_32B")
    with_bytes = all(c in names for c in sized)
    lines = ["# rocprofv3 counters per dispatch", "", "Command:", "", "```", cmd, "```", "",
             *([note, ""] if note else []),
             "Means per dispatch. GRBM_GUI_ACTIVE sums the cycles of the 8 XCDs, so the clock is "
             "GRBM_GUI_ACTIVE / 8 / duration. Matrix-core busy = SQ_VALU_MFMA_BUSY_CYCLES / "
             "(1024 SIMDs x GRBM_GUI_ACTIVE / 8): the share of the kernel's cycles an average "
             "SIMD's matrix core was busy.", "",
             *(["Read bytes = 128 TCC_EA0_RDREQ_128B + 64 TCC_EA0_RDREQ_64B + 32 "
                "TCC_EA0_RDREQ_32B (HBM read requests by size, summed over the L2 channels; no "
                "calibration factor).", ""] if with_bytes else []),
             "| kernel | grid | dispatches | avg us | " + " | ".join(names) +
             " | clock GHz | matrix-core busy |" + (" read bytes |" if with_bytes else ""),
             "|---|---|---|---|" + "---|" * len(names) + "---|---|" + ("---|" if with_bytes else "")]
    for sel in selects:
        name, grid = sel.rsplit(":", 1)
        grid = int(grid)
        keys = [k for k in vals if name in k[0] and k[1] == grid]
        if not keys:
            raise SystemExit(f"no dispatch of {name} with grid {grid}")
        agg = collections.defaultdict(list)
        ds = []
        for k in keys:
            for c, v in vals[k].items():
                agg[c] += v
            ds += list(durs[k].values())
        mean = {c: sum(v) / len(v) for c, v in agg.items()}
        dur_ns = sum(ds) / len(ds)
        grbm = mean.get("GRBM_GUI_ACTIVE")
        clock = f"{grbm / MI355X_XCDS / dur_ns:.2f}" if grbm else "-"
        busy = "-"
        if grbm and "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            busy = f"{mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (MI355X_SIMDS * grbm / MI355X_XCDS):.3f}"
        cells = " | ".join(f"{mean[c]:.4g}" if c in mean else "-" for c in names)
        rb = ""
        if with_bytes:
            rb = f" {128 * mean[sized[0]] + 64 * mean[sized[1]] + 32 * mean[sized[2]]:.4g} |"
        lines.append(f"| `{_short(keys[0][0])}` | {grid} | {len(ds)} | {dur_ns / 1e3:.2f} | "
                     f"{cells} | {clock} | {busy} |{rb}")
    return "\n".join(lines) + "\n"


def read_traffic(md_path: str, algorithmic: int):
    """Returns the stored traffic (bytes per call) if the decode sources and the workload's
    algorithmic bytes still match the ones the counters were taken with, else None."""
    if not os.path.exists(md_path):
        return None
    kv = {}
    for line in open(md_path, encoding="utf-8"):
        if ":" in line and not line.startswith(("|", "#", " ")):
            k, _, v = line.partition(":")
            kv[k.strip()] = v.strip()
    if kv.get("sources_sha256") != sources_sha256() or "traffic_bytes_per_call" not in kv:
        return None
    if kv.get("algorithmic_bytes_per_call") != str(algorithmic):
        return None
    return int(kv["traffic_bytes_per_call"])


def main():
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("trace_csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--note", default="")
    s.add_argument("-o", "--out", required=True)
    s.add_argument("--split", action="append", default=[])
    s.add_argument("--only", action="append", default=[])
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--select", action="append", required=True)
    t.add_argument("--algorithmic-bytes", type=int, required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--note", default="")
    t.add_argument("-o", "--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("pmc_csv")
    c.add_argument("--select", action="append", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--note", default="")
    c.add_argument("-o", "--out", required=True)
    a = p.parse_args()
    if a.what == "stats":
        text = stats(a.trace_csv, a.cmd, a.note, a.split, a.only)
    elif a.what == "counters":
        text = counters(a.pmc_csv, a.select, a.cmd, a.note)
    else:
        text = traffic(a.fetch_csv, a.write_csv, a.copy_bytes, a.select, a.algorithmic_bytes,
                       a.cmd, a.note)
    with open(a.out, "w", encoding="utf-8") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
