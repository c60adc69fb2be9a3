"""Summaries of rocprofv3 CSV output for this library's kernels.

    python prof_summary.py stats KERNEL_STATS_CSV --cmd "..." \\
            [--timed NAME:FIRST:COUNT] [--shapes NAME;NAME]
        per-kernel time table (the library's kernels first) from a
        ``rocprofv3 --kernel-trace --stats -f csv`` run; --timed adds the
        average of dispatches FIRST .. FIRST + COUNT - 1 of kernel NAME from
        the run's kernel trace (e.g. the launches a benchmark timed); --shapes
        splits the named kernels' dispatches by launch grid.

    python prof_summary.py traffic --fetch CSV --write CSV \\
            --copy-bytes N --kernel NAME --source FILE --cmd-fetch "..." --cmd-write "..."
        HBM bytes per launch of one kernel from a ``--pmc FETCH_SIZE`` run and a
        ``--pmc WRITE_SIZE`` run (counter values in KiB per dispatch).  Each
        counter is scaled by what it reads for a plain device copy of N bytes in
        the same run (N read, N written), and the result is tagged with the
        SHA-256 of the kernel's source file so that a reader can tell whether
        the figure still belongs to the current kernel.

    python prof_summary.py counters --csv CSV [--csv CSV ...] --cmd "..." [--cmd ...] \\
            --kernel NAME [--kernel NAME ...]
        per-dispatch averages of every counter of ``--pmc`` runs for the named
        kernels, one column per (kernel, launch grid).

Output is Markdown on stdout.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import statistics
import sys


def _short(name: str) -> str:
    name = name.replace("f4kv::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    if "(" in name:
        name = name[:name.index("(")]
    return name.replace("void ", "").strip()


def timed_window(trace_path: str, spec: str) -> str:
    """Average duration of dispatches FIRST .. FIRST + COUNT - 1 (in start order)
    of one kernel, from a kernel-trace CSV; spec = "NAME:FIRST:COUNT"."""
    name, first, count = spec.rsplit(":", 2)
    first, count = int(first), int(count)
    rows = [r for r in csv.DictReader(open(trace_path)) if name in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows[first:first + count]]
    if len(d) != count:
        raise SystemExit(f"only {len(d)} dispatches of {name!r} in that window")
    return (f"`{name}`, dispatches {first + 1} .. {first + count} of {len(rows)} in start order (the timed launches): "
            f"average {statistics.mean(d):.1f} us, min {min(d):.1f}, max {max(d):.1f}.")


def launch_shapes(trace_path: str, names) -> str:
    """Per-grid rows of the named kernels (one kernel serving two entry points,
    say), from a kernel-trace CSV."""
    groups = {}
    for r in csv.DictReader(open(trace_path)):
        if "f4kv::" not in r["Kernel_Name"] or _short(r["Kernel_Name"]) not in names:
            continue
        grid = tuple(int(r[f"Grid_Size_{a}"]) // max(1, int(r[f"Workgroup_Size_{a}"])) for a in "XYZ")
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault(_short(r["Kernel_Name"]), {}).setdefault(grid, []).append(d)
    lines = []
    for name, by_grid in sorted(groups.items()):
        for grid, d in sorted(by_grid.items(), key=lambda kv: -statistics.mean(kv[1])):
            lines.append(f"| `{name}` | {grid[0]} x {grid[1]} x {grid[2]} | {len(d)} | {statistics.mean(d):.1f} | "
                         f"{min(d):.1f} | {max(d):.1f} |")
    if not lines:
        return ""
    return "\n".join(["", "Launch grids (workgroups x, y, z) of " + ", ".join(f"`{n}`" for n in names)
                      + ", from the kernel trace:", "",
                      "| kernel | grid | calls | avg us | min us | max us |", "|---|---|---:|---:|---:|---:|"]
                     + lines)


def stats_table(path: str, cmd: str, timed: str = "", shapes=()) -> str:
    rows = list(csv.DictReader(open(path)))
    lines = ["# Kernel time summary", "", "Command:", "", "```", cmd, "```", "",
             "| kernel | calls | avg us | min us | max us | share of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    ours = [r for r in rows if "f4kv::" in r["Name"]]
    other = [r for r in rows if "f4kv::" not in r["Name"]]
    for r in ours + other[:5]:
        lines.append(f"| `{_short(r['Name'])[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.2f}% |")
    if len(other) > 5:
        lines.append(f"| ({len(other) - 5} more kernels of the harness) | | | | | |")
    trace = path.replace("kernel_stats.csv", "kernel_trace.csv")
    if shapes:
        lines.append(launch_shapes(trace, shapes))
    if timed:
        lines += ["", timed_window(trace, timed)]
    return "\n".join(lines) + "\n"


def _counter(path: str, counter: str):
    by_kernel = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        by_kernel.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return by_kernel


def _copy_value(by_kernel, nbytes: int) -> float:
    """Median counter value (KiB) of the copy dispatches of nbytes: the largest
    values among the blit/copy kernels."""
    cand = []
    for name, vals in by_kernel.items():
        if "copyBuffer" in name or "copy" in name.lower():
            cand.extend(vals)
    cand.sort(reverse=True)
    top = cand[:3]
    if not top:
        raise SystemExit("no copy dispatch found in the counter file")
    return statistics.median(top)


def _kernel_values(by_kernel, kernel: str):
    vals = []
    for name, v in by_kernel.items():
        if kernel in name:
            vals.extend(v)
    if not vals:
        raise SystemExit(f"kernel {kernel!r} not found in the counter file")
    return vals


def traffic(a) -> str:
    fetch = _counter(a.fetch, "FETCH_SIZE")
    write = _counter(a.write, "WRITE_SIZE")
    copy_kib = a.copy_bytes / 1024.0
    f_copy = _copy_value(fetch, a.copy_bytes)
    w_copy = _copy_value(write, a.copy_bytes)
    f_scale = copy_kib / f_copy
    w_scale = copy_kib / w_copy
    fk = _kernel_values(fetch, a.kernel)
    wk = _kernel_values(write, a.kernel)
    f_bytes = statistics.mean(fk) * f_scale * 1024.0
    w_bytes = statistics.mean(wk) * w_scale * 1024.0
    sha = hashlib.sha256(open(a.source, "rb").read()).hexdigest()
    out = [f"# HBM traffic of `{a.kernel}`", "",
           "Commands (FETCH_SIZE run, then WRITE_SIZE run):", "", "```", a.cmd_fetch, a.cmd_write, "```", "",
           f"Copy calibration: a device copy of {a.copy_bytes} bytes ({copy_kib:.0f} KiB read and written) "
           f"reads FETCH_SIZE = {f_copy:.1f} KiB and WRITE_SIZE = {w_copy:.1f} KiB per dispatch, so the "
           f"counters are scaled by {f_scale:.4f} (fetch) and {w_scale:.4f} (write).", "",
           "| counter | dispatches | mean KiB | min KiB | max KiB | scaled bytes per launch |",
           "|---|---:|---:|---:|---:|---:|",
           f"| FETCH_SIZE | {len(fk)} | {statistics.mean(fk):.1f} | {min(fk):.1f} | {max(fk):.1f} | {f_bytes:.0f} |",
           f"| WRITE_SIZE | {len(wk)} | {statistics.mean(wk):.1f} | {min(wk):.1f} | {max(wk):.1f} | {w_bytes:.0f} |",
           "",
           f"- fetch bytes per launch: {f_bytes:.0f}",
           f"- write bytes per launch: {w_bytes:.0f}",
           f"- traffic bytes per launch: {f_bytes + w_bytes:.0f}",
           f"- copy scale fetch: {f_scale:.6f}",
           f"- copy scale write: {w_scale:.6f}",
           f"- {a.source.split('/')[-1]} sha256: `{sha}`", ""]
    return "\n".join(out)


def counters(paths, cmds, kernels) -> str:
    """Per-dispatch averages of every counter in the given ``--pmc`` CSVs for
    each named kernel, one column per (kernel, launch grid)."""
    cols = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            short = _short(r["Kernel_Name"])
            if short not in kernels:
                continue
            grid = tuple(int(r.get(f"Grid_Size_{a}", r.get("Grid_Size", 0)) or 0) //
                         max(1, int(r.get(f"Workgroup_Size_{a}", r.get("Workgroup_Size", 1)) or 1)) for a in "XYZ") \
                if "Grid_Size_X" in r else (int(r.get("Grid_Size", 0)),)
            key = (short, grid)
            cols.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not cols:
        raise SystemExit("none of the kernels found in the counter files")
    names = sorted({c for v in cols.values() for c in v})
    keys = sorted(cols)
    head = ["# Counters per dispatch", "", "Commands (one counter group per pass):", "", "```", *cmds, "```", "",
            "| counter | " + " | ".join(f"`{k[0]}` grid {' x '.join(map(str, k[1]))}" for k in keys) + " |",
            "|---|" + "---:|" * len(keys)]
    rows = []
    disp = []
    for k in keys:
        n = max(len(v) for v in cols[k].values())
        disp.append(str(n))
    rows.append("| dispatches | " + " | ".join(disp) + " |")
    for c in names:
        vals = []
        for k in keys:
            d = cols[k].get(c)
            vals.append(f"{statistics.mean(d):,.0f}" if d else "")
        rows.append(f"| {c} | " + " | ".join(vals) + " |")
    return "\n".join(head + rows) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--timed", default="", help="NAME:FIRST:COUNT: also average these dispatches of NAME")
    s.add_argument("--shapes", default="", help="NAME[;NAME]: also list these kernels' dispatches per launch grid")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--source", required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--csv", action="append", required=True)
    c.add_argument("--cmd", action="append", required=True)
    c.add_argument("--kernel", action="append", required=True, help="short kernel name, e.g. 'decode_kernel<4, false>'")
    a = ap.parse_args(argv)
    if a.what == "stats":
        sys.stdout.write(stats_table(a.csv, a.cmd, a.timed, [n for n in a.shapes.split(";") if n]))
    elif a.what == "counters":
        sys.stdout.write(counters(a.csv, a.cmd, a.kernel))
    else:
        sys.stdout.write(traffic(a))


if __name__ == "__main__":
    main()
