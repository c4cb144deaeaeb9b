"""Summaries of rocprofv3 runs of bench.py, written as short text files.

Two products:

* ``<kernel-trace dir>`` (``rocprofv3 --kernel-trace --stats --output-format
  csv``) -> a markdown table of per-kernel calls and durations;
* two counter runs (``rocprofv3 --pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``
  of ``bench.py --copy-calibration MIB``) -> HBM bytes per dispatch of every
  kernel.  Each counter is scaled by the ratio of the known size of the
  calibration copy to what the same counter reads for that copy.  The table
  records a digest of the library sources, so a reader can tell whether the
  kernels have changed since the counters were taken.

* several counter runs (``rocprofv3 --pmc <SQ counters>``, one pass each) ->
  per-kernel averages per dispatch and derived ratios (instructions per wave,
  the share of wave lifetime spent waiting or issuing, LDS bank conflicts).

Usage::

    python -m integer_only_dnn_amd.prof_summary stats  --dir D --out profiles/x.md --cmd "..."
    python -m integer_only_dnn_amd.prof_summary traffic --fetch D1 --write D2 --copy-mib 256 \\
        --workload resnet18 --out profiles/y.txt --cmd "..." --cmd "..."
    python -m integer_only_dnn_amd.prof_summary counters --dir D1 --dir D2 --dir D3 \\
        --workload resnet50 --out profiles/z.md --cmd "..." --cmd "..."
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def source_digest() -> str:
    """sha256 over the library's kernel sources (name and content, sorted)."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(CSRC, "*.hip")) +
                       glob.glob(os.path.join(CSRC, "*.cpp"))):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    """'void ie::gemm_i8_kernel<1, 4, 1, 1, true, false>(ie::Operand, ...)' ->
    'gemm_i8_kernel<1, 4, 1, 1, true, false>'."""
    n = re.sub(r"\(.*$", "", name).replace("void ", "").strip()
    return n.replace("ie::", "")


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[-1]


def kernel_stats(trace_dir: str):
    path = _one(os.path.join(trace_dir, "**", "*kernel_stats.csv"))
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append({"name": short_name(r["Name"]), "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3, "total_ms": float(r["TotalDurationNs"]) / 1e6,
                         "pct": float(r["Percentage"]), "min_us": float(r["MinNs"]) / 1e3,
                         "max_us": float(r["MaxNs"]) / 1e3})
    return rows


def counter_per_kernel(pmc_dir: str):
    """{kernel: (dispatches, mean counter value per dispatch)} of a --pmc run."""
    path = _one(os.path.join(pmc_dir, "**", "*counter_collection.csv"))
    acc = defaultdict(lambda: [0, 0.0])
    grid = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            k = short_name(r["Kernel_Name"])
            if k == COPY_KERNEL:
                # keep the large calibration copy apart from small runtime copies
                g = int(r.get("Grid_Size", 0) or 0)
                k = f"{COPY_KERNEL}#grid{g}"
                grid[k] = g
            a = acc[k]
            a[0] += 1
            a[1] += float(r["Counter_Value"])
    return {k: (n, v / n) for k, (n, v) in acc.items()}


def _copy_entry(per):
    copies = [k for k in per if k.startswith(COPY_KERNEL)]
    if not copies:
        raise SystemExit("the counter run holds no calibration copy (run bench.py with --copy-calibration)")
    return max(copies, key=lambda k: per[k][1])


def write_stats(trace_dir: str, out: str, cmd: str, top: int = 25) -> None:
    rows = kernel_stats(trace_dir)
    lines = [f"# rocprofv3 kernel statistics: {os.path.splitext(os.path.basename(out))[0]}", "",
             "Command (run from /tmp with TMPDIR=/tmp; bench.py at the repository root):", "", "```",
             cmd, "```", "", f"Library source digest: {source_digest()}", "",
             "| kernel | calls | avg us | min us | max us | total ms | % |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows[:top]:
        lines.append(f"| `{r['name']}` | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                     f"{r['max_us']:.2f} | {r['total_ms']:.3f} | {r['pct']:.1f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_traffic(fetch_dir: str, write_dir: str, copy_mib: int, workload: str, out: str, cmds) -> None:
    fetch, write = counter_per_kernel(fetch_dir), counter_per_kernel(write_dir)
    copy_kib = copy_mib * 1024.0
    fk, wk = _copy_entry(fetch), _copy_entry(write)
    f_scale = copy_kib / fetch[fk][1]
    w_scale = copy_kib / write[wk][1]
    lines = [f"# HBM traffic per dispatch, workload {workload}",
             "# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two rocprofv3 --pmc runs, each scaled by",
             f"# (known size of the calibration copy, {copy_mib} MiB) / (the counter's reading for that copy).",
             f"# fetch scale {f_scale:.4f}, write scale {w_scale:.4f}"]
    lines += [f"# command: {c}" for c in cmds]
    lines += [f"source_digest {source_digest()}", "# kernel | dispatches | fetch_bytes | write_bytes"]
    for k in sorted(fetch):
        if k.startswith(COPY_KERNEL) or k not in write:
            continue
        n, fv = fetch[k]
        lines.append(f"{k} | {n} | {fv * 1024 * f_scale:.0f} | {write[k][1] * 1024 * w_scale:.0f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_traffic(path: str):
    """(source digest, {kernel: (fetch_bytes, write_bytes)}) of a traffic table."""
    digest, table = None, {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("source_digest "):
                digest = line.split()[1]
                continue
            parts = [p.strip() for p in line.split("|")]
            if len(parts) == 4:
                table[parts[0]] = (float(parts[2]), float(parts[3]))
    return digest, table


def counters_per_kernel(dirs):
    """{kernel: {counter: mean value per dispatch}} over several --pmc runs,
    and {kernel: dispatches}."""
    acc = defaultdict(lambda: defaultdict(lambda: [0, 0.0]))
    disp = defaultdict(set)
    for d in dirs:
        path = _one(os.path.join(d, "**", "*counter_collection.csv"))
        with open(path) as f:
            for r in csv.DictReader(f):
                k = short_name(r["Kernel_Name"])
                a = acc[k][r["Counter_Name"]]
                a[0] += 1
                a[1] += float(r["Counter_Value"])
                disp[k].add((d, r.get("Dispatch_Id", r.get("Correlation_Id", ""))))
    return ({k: {c: v / n for c, (n, v) in cs.items()} for k, cs in acc.items()},
            {k: len(v) // max(1, len(dirs)) for k, v in disp.items()})


def write_counters(dirs, workload: str, out: str, cmds, top: int = 16) -> None:
    per, ndisp = counters_per_kernel(dirs)

    def g(cs, name):
        return cs.get(name)

    def ratio(a, b, scale=1.0):
        return f"{100.0 * scale * a / b:.1f}" if a is not None and b else "-"

    def per_wave(cs, name):
        v, w = g(cs, name), g(cs, "SQ_WAVES")
        return f"{v / w:.0f}" if v is not None and w else "-"

    rows = sorted(per.items(), key=lambda kv: -(kv[1].get("SQ_WAVE_CYCLES", 0.0) * ndisp.get(kv[0], 1)))
    lines = [f"# Hardware counters per kernel: {workload}", "",
             "Commands (run from /tmp with TMPDIR=/tmp; bench.py at the repository root; one pass per counter "
             "set):", "", "```"] + list(cmds) + ["```", "",
             f"Library source digest: {source_digest()}", "",
             "Per dispatch, averaged over dispatches.  Columns: waves; instructions per wave (VALU, MFMA, LDS, "
             "vector-memory reads); `wait%` = SQ_WAIT_ANY / SQ_WAVE_CYCLES (wave lifetime waiting on a memory "
             "or LDS counter); `valu%`, `lds%` = SQ_ACTIVE_INST_VALU, SQ_ACTIVE_INST_LDS over SQ_WAVE_CYCLES "
             "(lifetime issuing); `mfma%` = SQ_VALU_MFMA_BUSY_CYCLES / (SQ_BUSY_CU_CYCLES x 4 SIMDs), the "
             "share of busy-CU cycles the matrix cores work; `bank%` = SQ_LDS_BANK_CONFLICT / "
             "SQ_LDS_IDX_ACTIVE.", "",
             "| kernel | disp | waves | VALU/w | MFMA/w | LDS/w | VMEMrd/w | wait% | valu% | lds% | mfma% | bank% |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for k, cs in rows[:top]:
        wc = g(cs, "SQ_WAVE_CYCLES")
        lines.append(
            f"| `{k}` | {ndisp.get(k, 0)} | {g(cs, 'SQ_WAVES') or 0:.0f} | {per_wave(cs, 'SQ_INSTS_VALU')} | "
            f"{per_wave(cs, 'SQ_INSTS_MFMA')} | {per_wave(cs, 'SQ_INSTS_LDS')} | {per_wave(cs, 'SQ_INSTS_VMEM_RD')} | "
            f"{ratio(g(cs, 'SQ_WAIT_ANY'), wc)} | {ratio(g(cs, 'SQ_ACTIVE_INST_VALU'), wc)} | "
            f"{ratio(g(cs, 'SQ_ACTIVE_INST_LDS'), wc)} | "
            f"{ratio(g(cs, 'SQ_VALU_MFMA_BUSY_CYCLES'), g(cs, 'SQ_BUSY_CU_CYCLES'), 0.25)} | "
            f"{ratio(g(cs, 'SQ_LDS_BANK_CONFLICT'), g(cs, 'SQ_LDS_IDX_ACTIVE'))} |")
    lines += ["", "Raw means per dispatch:", ""]
    names = sorted({c for cs in per.values() for c in cs})
    lines.append("| kernel | " + " | ".join(names) + " |")
    lines.append("|---|" + "---:|" * len(names))
    for k, cs in rows[:top]:
        lines.append(f"| `{k}` | " + " | ".join(f"{cs[c]:.4g}" if c in cs else "-" for c in names) + " |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--dir", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--cmd", action="append", default=[])
    c = sub.add_parser("counters")
    c.add_argument("--dir", action="append", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--cmd", action="append", default=[])
    c.add_argument("--top", type=int, default=16)
    a = ap.parse_args()
    if a.what == "stats":
        write_stats(a.dir, a.out, a.cmd)
    elif a.what == "counters":
        write_counters(a.dir, a.workload, a.out, a.cmd, a.top)
    else:
        write_traffic(a.fetch, a.write, a.copy_mib, a.workload, a.out, a.cmd)


if __name__ == "__main__":
    main()
