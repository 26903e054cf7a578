"""Short text summaries of rocprofv3 output, for the profiles/ folder.

Kernel durations (from ``rocprofv3 --kernel-trace --stats --output-format csv``)::

    python -m memory_bound_transformer_decode_amd.profile_summary stats DIR \
        --command "<the rocprofv3 command>" [--top 12] [--match dec::] > profiles/<...>.md

Counters of any --pmc run, as the mean per dispatch for each kernel::

    python -m memory_bound_transformer_decode_amd.profile_summary counters DIR \
        --command "<the rocprofv3 command>" [--match dec::] > profiles/<...>.md

HBM traffic of one kernel per dispatch, from two counter runs of the benchmark
(``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``) and two of a device-to-device copy of
known size (the same counters; they give the bytes-per-reported-unit factors)::

    python -m memory_bound_transformer_decode_amd.profile_summary traffic \
        --fetch DIR1 --write DIR2 --copy-fetch DIR3 --copy-write DIR4 --copy-bytes N \
        --kernel SUBSTRING --commands "<...>" > profiles/<kernel>_<workload>_traffic.txt

Host time of the library's calls, from the roctx ranges it opens around them
(``rocprofv3 --marker-trace --output-format csv``), skipping each name's first
``--skip`` calls (the graph captures)::

    python -m memory_bound_transformer_decode_amd.profile_summary markers DIR \
        --command "<the rocprofv3 command>" [--skip 1] > profiles/<...>_markers.md

The traffic file ends with ``source_sha256`` of the kernel family's sources (``--family``
gemv, gemm or attn), which bench.py compares with the tree it runs from: counters taken
on another version of the kernel are not reported.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import sys
from typing import Dict, List

# sources of each kernel family whose traffic is summarized
KERNEL_SOURCES = {
    "gemv": ("csrc/matmul.hip", "csrc/gemv_norm.h", "csrc/epilogue.h", "csrc/common.h", "csrc/kernels.h"),
    "gemm": ("csrc/gemm_mfma.hip", "csrc/epilogue.h", "csrc/common.h", "csrc/kernels.h"),
    "attn": ("csrc/attention.hip", "csrc/attn_unit.h", "csrc/common.h", "csrc/kernels.h"),
}


def kernel_source_sha256(family: str = "gemv") -> str:
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        with open(os.path.join(here, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[-1]


def _col(row: Dict[str, str], *names: str) -> str:
    low = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    raise KeyError(f"none of {names} in {list(row)}")


def stats(args) -> None:
    path = _find(args.dir, "kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    if args.match:
        # the share column stays a share of all GPU time, set-up kernels included
        rows = [r for r in rows if args.match in _col(r, "Name", "KernelName")]
    rows.sort(key=lambda r: -float(_col(r, "TotalDurationNs")))
    print("# Kernel durations (rocprofv3 --kernel-trace --stats)\n")
    print(f"Command: `{args.command}`\n")
    print("| kernel | calls | average us | min us | max us | share % |")
    print("|---|---|---|---|---|---|")
    for r in rows[: args.top]:
        name = _col(r, "Name", "KernelName")
        print(f"| `{name[:110]}` | {_col(r, 'Calls')} | {float(_col(r, 'AverageNs')) / 1e3:.2f} | "
              f"{float(_col(r, 'MinNs')) / 1e3:.2f} | {float(_col(r, 'MaxNs')) / 1e3:.2f} | "
              f"{float(_col(r, 'Percentage')):.2f} |")


def _counter(d: str, counter: str, kernel: str) -> List[float]:
    path = _find(d, "counter_collection.csv")
    vals = []
    for r in csv.DictReader(open(path)):
        if _col(r, "Counter_Name", "CounterName") != counter:
            continue
        if kernel in _col(r, "Kernel_Name", "KernelName"):
            vals.append(float(_col(r, "Counter_Value", "CounterValue")))
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel!r} in {path}")
    return vals


def counters(args) -> None:
    """Mean per dispatch of every counter of a --pmc run, per kernel."""
    path = _find(args.dir, "counter_collection.csv")
    acc: Dict[tuple, List[float]] = {}
    for r in csv.DictReader(open(path)):
        name = _col(r, "Kernel_Name", "KernelName")
        if args.match not in name:
            continue
        key = (name, _col(r, "Counter_Name", "CounterName"))
        acc.setdefault(key, []).append(float(_col(r, "Counter_Value", "CounterValue")))
    names = sorted({k for k, _ in acc})
    ctrs = sorted({c for _, c in acc})
    print("# Counters per dispatch (rocprofv3 --pmc), mean over dispatches\n")
    print(f"Command: `{args.command}`\n")
    print("| kernel | dispatches | " + " | ".join(ctrs) + " |")
    print("|---|---|" + "---|" * len(ctrs))
    for n in names:
        vals = [acc.get((n, c), []) for c in ctrs]
        print(f"| `{n[:90]}` | {max(len(v) for v in vals)} | " +
              " | ".join(f"{sum(v) / len(v):.4g}" if v else "" for v in vals) + " |")


def traffic(args) -> None:
    kib = 1024.0
    f = _counter(args.fetch, "FETCH_SIZE", args.kernel)
    w = _counter(args.write, "WRITE_SIZE", args.kernel)
    cf = _counter(args.copy_fetch, "FETCH_SIZE", args.copy_kernel)
    cw = _counter(args.copy_write, "WRITE_SIZE", args.copy_kernel)
    # the copy moves copy_bytes in and copy_bytes out: bytes per reported KiB
    ffac = args.copy_bytes / (max(cf) * kib)
    wfac = args.copy_bytes / (max(cw) * kib)
    fetch = sum(f) / len(f) * kib * ffac
    write = sum(w) / len(w) * kib * wfac
    print("# HBM traffic per dispatch (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)")
    print(f"# commands: {args.commands}")
    print(f"kernel: {args.kernel}")
    print(f"family: {args.family}")
    print(f"dispatches: {len(f)} (fetch), {len(w)} (write)")
    print(f"fetch_kib_per_dispatch: {sum(f) / len(f):.1f}")
    print(f"write_kib_per_dispatch: {sum(w) / len(w):.1f}")
    print(f"copy_bytes: {args.copy_bytes}")
    print(f"copy_fetch_kib: {max(cf):.1f}")
    print(f"copy_write_kib: {max(cw):.1f}")
    print(f"fetch_factor: {ffac:.4f}")
    print(f"write_factor: {wfac:.4f}")
    print(f"fetch_bytes_per_dispatch: {fetch:.0f}")
    print(f"write_bytes_per_dispatch: {write:.0f}")
    print(f"traffic_bytes_per_dispatch: {fetch + write:.0f}")
    print(f"source_sha256: {kernel_source_sha256(args.family)}")


def markers(args) -> None:
    path = _find(args.dir, "marker_api_trace.csv")
    spans: Dict[str, List[float]] = {}
    for r in csv.DictReader(open(path)):
        name = _col(r, "Function", "Message")
        d = (int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) / 1e3
        spans.setdefault(name, []).append(d)
    print("# Host time of the library's calls (roctx ranges, rocprofv3 --marker-trace)\n")
    print(f"Command: `{args.command}`\n")
    print(f"The first {args.skip} call(s) of each name (graph capture) are left out.\n")
    print("| range | calls | mean us | median us | min us | max us |")
    print("|---|---|---|---|---|---|")
    for name in sorted(spans):
        d = sorted(spans[name][args.skip:]) if len(spans[name]) > args.skip else []
        if not d:
            continue
        print(f"| `{name}` | {len(d)} | {sum(d) / len(d):.1f} | {d[len(d) // 2]:.1f} | {d[0]:.1f} | {d[-1]:.1f} |")


def read_traffic(path: str) -> Dict[str, str]:
    out = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--command", required=True)
    s.add_argument("--top", type=int, default=12)
    s.add_argument("--match", default="", help="keep only kernels whose name contains this text")
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--command", required=True)
    c.add_argument("--match", default="", help="keep only kernels whose name contains this text")
    t = sub.add_parser("traffic")
    for name in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--kernel", "--commands"):
        t.add_argument(name, required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--copy-kernel", default="copyBuffer")
    t.add_argument("--family", choices=sorted(KERNEL_SOURCES), default="gemv")
    m = sub.add_parser("markers")
    m.add_argument("dir")
    m.add_argument("--command", required=True)
    m.add_argument("--skip", type=int, default=1, help="leave out each range's first calls")
    args = ap.parse_args(argv)
    {"stats": stats, "counters": counters, "traffic": traffic, "markers": markers}[args.cmd](args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
