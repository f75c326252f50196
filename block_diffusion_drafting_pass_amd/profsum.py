"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m block_diffusion_drafting_pass_amd.profsum trace KERNEL_STATS_CSV OUT_TXT --cmd "..."
    python -m block_diffusion_drafting_pass_amd.profsum traffic FETCH_CSV WRITE_CSV OUT_TXT \
        --kernel SUBSTRING --copy-bytes N --cmd "..." --cmd "..."

``trace`` lists every kernel of a ``--kernel-trace --stats`` run (calls,
average / min / max duration, share of GPU time).  ``traffic`` takes two
``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs (KiB per dispatch), finds the
plain device-to-device copy of ``--copy-bytes`` bytes that bench.py makes
before its timed region, derives from it the factor between what each counter
reads and the bytes actually moved, and applies that factor to the chosen
kernel.  The summary records a hash of the kernel sources so that bench.py
only reports the traffic while the kernels are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics
from typing import List

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("csrc/kernels.hip", "csrc/kernels.h")


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def trace(stats_csv: str, out: str, cmds: List[str]) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# rocprofv3 kernel trace summary", "# command(s):"]
    lines += [f"#   {c}" for c in cmds]
    lines.append(f"# kernel sources sha256: {kernel_sources_sha256()}")
    lines.append(f"{'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'total_ms':>9} {'pct':>6}  kernel")
    for r in rows:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                     f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['TotalDurationNs']) / 1e6:9.3f} "
                     f"{float(r['Percentage']):6.2f}  {r['Name'][:150]}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_dispatch(path: str, match) -> List[float]:
    return [float(r["Counter_Value"]) for r in csv.DictReader(open(path)) if match(r)]


def traffic(fetch_csv: str, write_csv: str, out: str, kernel: str, copy_bytes: int, cmds: List[str]) -> None:
    copy_grid = None
    for r in csv.DictReader(open(fetch_csv)):
        if "copyBuffer" in r["Kernel_Name"]:
            g = int(r["Grid_Size"])
            copy_grid = g if copy_grid is None else max(copy_grid, g)
    is_copy = lambda r: "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) == copy_grid  # noqa: E731
    is_kern = lambda r: kernel in r["Kernel_Name"]  # noqa: E731
    cf, cw = _per_dispatch(fetch_csv, is_copy), _per_dispatch(write_csv, is_copy)
    kf, kw = _per_dispatch(fetch_csv, is_kern), _per_dispatch(write_csv, is_kern)
    if not (cf and cw and kf and kw):
        raise SystemExit("copy kernel or target kernel not found in the counter files")
    name = next(r["Kernel_Name"] for r in csv.DictReader(open(fetch_csv)) if is_kern(r))
    kib = copy_bytes / 1024.0
    fetch_scale = kib / statistics.median(cf)
    write_scale = kib / statistics.median(cw)
    f_kib, w_kib = statistics.median(kf), statistics.median(kw)
    total = (f_kib * fetch_scale + w_kib * write_scale) * 1024.0
    lines = ["# HBM traffic of one kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch)",
             "# command(s):"]
    lines += [f"#   {c}" for c in cmds]
    lines += [
        f"kernel: {name}",
        f"kernel_sources_sha256: {kernel_sources_sha256()}",
        f"dispatches: {len(kf)}",
        f"fetch_kib_per_dispatch: {f_kib:.1f}",
        f"write_kib_per_dispatch: {w_kib:.1f}",
        f"copy_kernel: __amd_rocclr_copyBuffer, grid {copy_grid}, {copy_bytes} bytes read and written",
        f"copy_fetch_kib: {statistics.median(cf):.1f}",
        f"copy_write_kib: {statistics.median(cw):.1f}",
        f"fetch_scale: {fetch_scale:.4f}",
        f"write_scale: {write_scale:.4f}",
        f"traffic_bytes_per_dispatch: {total:.0f}",
    ]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_traffic(path: str):
    """(traffic_bytes_per_dispatch, kernel_sources_sha256) from a traffic summary, or None."""
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        if ln.startswith("#") or ":" not in ln:
            continue
        k, v = ln.split(":", 1)
        kv[k.strip()] = v.strip()
    try:
        return float(kv["traffic_bytes_per_dispatch"]), kv["kernel_sources_sha256"]
    except KeyError:
        return None


def main(argv=None) -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("out")
    t.add_argument("--cmd", action="append", default=[])
    p = sub.add_parser("traffic")
    p.add_argument("fetch_csv")
    p.add_argument("write_csv")
    p.add_argument("out")
    p.add_argument("--kernel", required=True)
    p.add_argument("--copy-bytes", type=int, default=1 << 30)
    p.add_argument("--cmd", action="append", default=[])
    a = ap.parse_args(argv)
    if a.mode == "trace":
        trace(a.stats_csv, a.out, a.cmd)
    else:
        traffic(a.fetch_csv, a.write_csv, a.out, a.kernel, a.copy_bytes, a.cmd)


if __name__ == "__main__":
    main()
