"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m sparse_long_sequence_amd.profsum traffic --fetch DIR --write DIR --kernel SUB \\
        [--kernel SUB ...] --calib-mib N --alg-bytes B --title T --cmd C [--cmd C ...] \\
        [--sources FILE ...]
    python -m sparse_long_sequence_amd.profsum counters --dir DIR --kernel SUB [--kernel SUB ...] \\
        --title T --cmd C [--sources FILE ...]
    python -m sparse_long_sequence_amd.profsum trace --dir DIR --kernel SUB [--last N] \\
        --title T --cmd C [--sources FILE ...]

DIR is a rocprofv3 output directory (``-d DIR --output-format csv``); the CSV files are
found below it.  Kernels are selected by a substring of their (mangled or demangled)
name; ``--note`` adds lines of explanation to the header.  ``traffic`` turns the per-dispatch FETCH_SIZE and WRITE_SIZE counters (KiB) of
two runs into bytes per launch, each scaled by what the same counter reads for the
plain elementwise copy (``torch.mul(src, 1.0, out=dst)``) of known size the measured
program ran at its end (``--calibrate-copy-mb``); with ``--trace DIR`` (a kernel-trace
run of the same program) it also gives each kernel's mean duration and the counted
bytes per second.  ``--sources`` lists the files the
measured kernels are built from; their sha256 (first 16 hex digits) is written into the
summary, so a reader (bench.py's ``stored_traffic``) can tell whether it still matches
the sources.  The summary goes to stdout.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_KERNEL = "AUnaryFunctor"   # torch's elementwise kernel of the calibration copy (x * 1.0)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _rows(d: str, suffix: str):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} below {d}")
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def _match(name: str, sub: str) -> bool:
    return sub in name


def counter_means(d: str, kernel: str):
    """{counter: (mean per dispatch, dispatches)} of the dispatches whose name holds kernel."""
    per = {}
    for r in _rows(d, "counter_collection.csv"):
        if not _match(r["Kernel_Name"], kernel):
            continue
        key = (r["Counter_Name"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
        per.setdefault(r["Counter_Name"], {}).setdefault(key[1], 0.0)
        per[r["Counter_Name"]][key[1]] += float(r["Counter_Value"])
    return {c: (statistics.fmean(v.values()), len(v)) for c, v in per.items()}


def kernel_names(d: str, suffix: str, sub: str):
    return sorted({r["Kernel_Name"] for r in _rows(d, suffix) if _match(r["Kernel_Name"], sub)})


def _header(title: str, cmds, sources, notes=()):
    lines = [f"# {title}", "#", "# Commands (each a run of its own, from /tmp with TMPDIR=/tmp; "
             "R = repository root):"]
    lines += [f"#   {c}" for c in cmds]
    if sources:
        lines += ["#", f"# kernel sources: {' '.join(sources)}"]
    if notes:
        lines += ["#"] + [f"# {n}" for n in notes]
    return lines


def cmd_traffic(a):
    out = _header(a.title, a.cmd, a.sources, a.note)
    fetch_copy = counter_means(a.fetch, COPY_KERNEL).get("FETCH_SIZE")
    write_copy = counter_means(a.write, COPY_KERNEL).get("WRITE_SIZE")
    if not fetch_copy or not write_copy:
        raise SystemExit("calibration copy kernel not found in the counter runs")
    mib_kib = a.calib_mib * 1024.0
    f_scale = mib_kib / fetch_copy[0]
    w_scale = mib_kib / write_copy[0]
    out += ["#", f"# Calibration: one plain elementwise copy (fp32 x 1.0) that reads {a.calib_mib} "
            f"MiB and writes {a.calib_mib} MiB.",
            f"#   FETCH_SIZE of that kernel: {fetch_copy[0]:.1f} KiB -> scale {f_scale:.4f}",
            f"#   WRITE_SIZE of that kernel: {write_copy[0]:.1f} KiB -> scale {w_scale:.4f}", "#"]
    total = None
    trace = _rows(a.trace, "kernel_trace.csv") if a.trace else None
    for k in a.kernel:
        fm = counter_means(a.fetch, k).get("FETCH_SIZE")
        wm = counter_means(a.write, k).get("WRITE_SIZE")
        if not fm or not wm:
            raise SystemExit(f"kernel {k!r} not found in the counter runs")
        fb = fm[0] * 1024.0 * f_scale
        wb = wm[0] * 1024.0 * w_scale
        names = kernel_names(a.fetch, "counter_collection.csv", k)
        out += [f"# {k}: {len(names)} instantiation(s), {fm[1]} / {wm[1]} dispatches",
                f"#   FETCH_SIZE {fm[0]:.1f} KiB raw -> {fb / 1e6:.4f} MB scaled",
                f"#   WRITE_SIZE {wm[0]:.1f} KiB raw -> {wb / 1e6:.4f} MB scaled"]
        if trace is not None:
            d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace
                 if _match(r["Kernel_Name"], k)]
            if d:
                mean = statistics.fmean(d)
                out += [f"#   duration (kernel trace, {len(d)} dispatches): mean {mean:.0f} ns "
                        f"-> {(fb + wb) / mean:.1f} GB/s counted ({100.0 * (fb + wb) / mean / 8000.0:.1f} % "
                        f"of 8 TB/s)"]
        if total is None:
            total = (k, fb, wb)
    k, fb, wb = total
    if a.alg_bytes:
        out += [f"#   algorithmic bytes per launch: {a.alg_bytes / 1e6:.4f} MB -> measured / "
                f"algorithmic = {(fb + wb) / a.alg_bytes:.3f}"]
    out += [f"kernel: {k}", f"workload: {a.workload}"]
    if a.sources:
        out += [f"kernel_source_sha256_16: {source_hash(a.sources)}"]
    out += [f"fetch_bytes_per_launch: {fb:.0f}", f"write_bytes_per_launch: {wb:.0f}",
            f"hbm_bytes_per_launch: {fb + wb:.0f}"]
    print("\n".join(out))


def cmd_counters(a):
    out = _header(a.title, a.cmd, a.sources, a.note)
    for k in a.kernel:
        m = counter_means(a.dir, k)
        if not m:
            raise SystemExit(f"kernel {k!r} not found")
        n = max(v[1] for v in m.values())
        out += [f"# {k}: mean per dispatch over {n} dispatches"]
        out += [f"{k} {c}: {v[0]:.6g}" for c, v in sorted(m.items())]
    if a.sources:
        out += [f"kernel_source_sha256_16: {source_hash(a.sources)}"]
    print("\n".join(out))


def cmd_trace(a):
    out = _header(a.title, a.cmd, a.sources, a.note)
    rows = _rows(a.dir, "kernel_trace.csv")
    for k in a.kernel:
        d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows
             if _match(r["Kernel_Name"], k)]
        if not d:
            raise SystemExit(f"kernel {k!r} not found")
        last = d[-a.last:] if a.last else d
        out += [f"# {k}: {len(d)} dispatches; the last {len(last)}: mean {statistics.fmean(last):.0f} ns, "
                f"median {statistics.median(last):.0f} ns, min {min(last)} ns, max {max(last)} ns"]
    stats = _rows(a.dir, "kernel_stats.csv")
    out += ["#", "# kernel_stats.csv:"]
    cols = list(stats[0].keys())
    out += [",".join(f'"{c}"' for c in cols)]
    out += [",".join(str(r[c]) for c in cols) for r in stats]
    if a.sources:
        out += ["#", f"kernel_source_sha256_16: {source_hash(a.sources)}"]
    print("\n".join(out))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="mode", required=True)
    for name in ("traffic", "counters", "trace"):
        p = sub.add_parser(name)
        p.add_argument("--kernel", action="append", required=True)
        p.add_argument("--title", required=True)
        p.add_argument("--cmd", action="append", default=[])
        p.add_argument("--sources", nargs="*", default=[])
        p.add_argument("--note", action="append", default=[],
                       help="a line of explanation for the summary's header (repeatable)")
        if name == "traffic":
            p.add_argument("--fetch", required=True)
            p.add_argument("--write", required=True)
            p.add_argument("--calib-mib", type=float, required=True)
            p.add_argument("--alg-bytes", type=float, default=0.0)
            p.add_argument("--workload", default="")
            p.add_argument("--trace", default="")
        else:
            p.add_argument("--dir", required=True)
        if name == "trace":
            p.add_argument("--last", type=int, default=0)
    a = ap.parse_args(argv)
    {"traffic": cmd_traffic, "counters": cmd_counters, "trace": cmd_trace}[a.mode](a)


if __name__ == "__main__":
    sys.exit(main())
