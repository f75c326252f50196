"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m block_diffusion_drafting_pass_amd.profsum trace KERNEL_STATS_CSV OUT_TXT --cmd "..."
    python -m block_diffusion_drafting_pass_amd.profsum traffic FETCH_CSV WRITE_CSV OUT_TXT \
        --kernel SUBSTRING --copy-bytes N --cmd "..." --cmd "..."
    python -m block_diffusion_drafting_pass_amd.profsum counters PMC_CSV OUT_TXT [--simds N] --cmd "..."
    python -m block_diffusion_drafting_pass_amd.profsum kernel OUT_TXT PMC_CSV [PMC_CSV ...] --kernel SUBSTRING --cmd "..."

``trace`` lists every kernel of a ``--kernel-trace --stats`` run (calls,
average / min / max duration, share of GPU time).  ``traffic`` takes two
``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs (KiB per dispatch), finds the
plain device-to-device copy of ``--copy-bytes`` bytes that bench.py makes
before its timed region, derives from it the factor between what each counter
reads and the bytes actually moved, and applies that factor to the chosen
kernel.  ``counters`` takes one ``--pmc SQ_INSTS_VALU_MFMA_MOPS_BF16
SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE`` run and sums, per draft pass, the
bf16 matrix-core flops the kernels executed (hi/lo products and padding rows
included) and the share of SIMD cycles the matrix cores were busy.
``kernel`` lists the counters of one kernel per dispatch and per wave.  The
summaries record a hash of the kernel sources so that bench.py only reports
their figures while the kernels are unchanged.
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


def _is_lm_head(name: str) -> bool:
    # the LM head is the GEMM instance with an argmax epilogue (first template
    # argument 1, greedy, or 3, sampled)
    return any(f"{k}<{e}," in name for k in ("k_skinny", "k_gemm_dl") for e in (1, 3))


def _agent_gpu(csv_path: str):
    """(SIMDs, XCDs) of the GPU from the run_agent_info.csv beside a counter file, or None."""
    path = os.path.join(os.path.dirname(csv_path), "run_agent_info.csv")
    if not os.path.exists(path):
        return None
    for r in csv.DictReader(open(path)):
        if r.get("Agent_Type") == "GPU":
            return int(r["Simd_Count"]), int(r["Num_Xcc"])
    return None


def counters(csv_path: str, out: str, cmds: List[str], simds: int, xcds: int) -> None:
    """Executed matrix-core work per draft pass from one --pmc run with
    SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE.
    A pass is every library kernel dispatched after one LM-head dispatch up
    to and including the next (setup work before the first LM head, such as
    the context ingest and the weight packing, is left out); figures are
    averages over those passes.  The one-time weight packing is left out
    wherever it falls.  rocprofv3 sums GRBM_GUI_ACTIVE over the XCDs, so the
    GPU's active cycles are that sum over the XCD count."""
    got = _agent_gpu(csv_path)
    if got is not None:
        simds, xcds = got
    disp = {}
    for r in csv.DictReader(open(csv_path)):
        d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "c": {},
                                                     "t": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    order = [disp[k] for k in sorted(disp)
             if "dflash::" in disp[k]["name"] and "k_pack_weights" not in disp[k]["name"]]
    heads = [i for i, d in enumerate(order) if _is_lm_head(d["name"])]
    if len(heads) < 2:
        raise SystemExit("fewer than two LM-head dispatches: no whole pass in the counter file")
    passes = len(heads) - 1
    per = {}
    for d in order[heads[0] + 1:heads[-1] + 1]:
        e = per.setdefault(d["name"], {"n": 0, "mops": 0.0, "busy": 0.0, "active": 0.0, "t": 0})
        e["n"] += 1
        e["mops"] += d["c"].get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        e["busy"] += d["c"].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        e["active"] += d["c"].get("GRBM_GUI_ACTIVE", 0.0) / xcds
        e["t"] += d["t"]
    tot_flops = sum(e["mops"] for e in per.values()) * 512.0 / passes
    tot_busy = sum(e["busy"] for e in per.values())
    tot_active = sum(e["active"] for e in per.values())
    tot_t = sum(e["t"] for e in per.values()) / passes
    lines = ["# executed matrix-core work of one draft pass from rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 "
             "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE",
             "# (bf16 MFMA flops = MOPS x 512; MFMA busy = busy cycles / (active cycles x SIMDs), the active",
             "# cycles being GRBM_GUI_ACTIVE summed over the XCDs divided by their count)",
             "# command(s):"]
    lines += [f"#   {c}" for c in cmds]
    lines += [f"kernel_sources_sha256: {kernel_sources_sha256()}",
              f"passes: {passes}",
              f"simds: {simds}",
              f"xcds: {xcds}",
              f"exec_bf16_flops_per_pass: {tot_flops:.6e}",
              f"mfma_busy_pass: {tot_busy / max(tot_active * simds, 1.0):.4f}",
              f"profiled_kernel_us_per_pass: {tot_t / 1e3:.1f}",
              f"{'per_pass':>8} {'exec_GFLOP':>11} {'busy':>6} {'us':>8}  kernel"]
    for name, e in sorted(per.items(), key=lambda kv: -kv[1]["mops"]):
        lines.append(f"{e['n'] / passes:8.1f} {e['mops'] * 512.0 / passes / 1e9:11.2f} "
                     f"{e['busy'] / max(e['active'] * simds, 1.0):6.3f} {e['t'] / passes / 1e3:8.1f}  {name[:140]}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def kernel_counters(csv_paths: List[str], out: str, kernel: str, cmds: List[str]) -> None:
    """Average counters per dispatch (and per wave) of every kernel whose name
    contains `kernel`, from one or more --pmc runs of the same workload."""
    lines = ["# rocprofv3 counters per dispatch of one kernel (averages over its dispatches; per wave = per"
             " dispatch / waves launched)", "# command(s):"]
    lines += [f"#   {c}" for c in cmds]
    lines.append(f"kernel_sources_sha256: {kernel_sources_sha256()}")
    for path in csv_paths:
        disp = {}
        for r in csv.DictReader(open(path)):
            if kernel not in r["Kernel_Name"]:
                continue
            d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "c": {},
                                                         "grid": int(r["Grid_Size"]), "wg": int(r["Workgroup_Size"]),
                                                         "t": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if not disp:
            raise SystemExit(f"no dispatch of {kernel} in {path}")
        ds = list(disp.values())
        waves = ds[0]["grid"] / 64
        lines.append(f"kernel: {ds[0]['name'][:160]}")
        lines.append(f"dispatches: {len(ds)}  grid threads: {ds[0]['grid']}  workgroup: {ds[0]['wg']}  "
                     f"profiled us per dispatch: {sum(d['t'] for d in ds) / len(ds) / 1e3:.2f}")
        for name in sorted(ds[0]["c"]):
            v = sum(d["c"].get(name, 0.0) for d in ds) / len(ds)
            lines.append(f"{name}: {v:.1f}  per wave {v / waves:.1f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_counters(path: str):
    """(exec_bf16_flops_per_pass, mfma_busy_pass, kernel_sources_sha256) from a counters summary, or None."""
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        if ln.startswith("#") or ":" not in ln:
            continue
        k, v = ln.split(":", 1)
        kv[k.strip()] = v.strip()
    try:
        return float(kv["exec_bf16_flops_per_pass"]), float(kv["mfma_busy_pass"]), kv["kernel_sources_sha256"]
    except KeyError:
        return None


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
    c = sub.add_parser("counters")
    c.add_argument("pmc_csv")
    c.add_argument("out")
    c.add_argument("--simds", type=int, default=1024, help="SIMDs of the GPU (MI355X: 256 CUs x 4), if the "
                   "run_agent_info.csv beside the counter file does not give them")
    c.add_argument("--xcds", type=int, default=8, help="XCDs of the GPU (MI355X: 8), likewise")
    c.add_argument("--cmd", action="append", default=[])
    k = sub.add_parser("kernel")
    k.add_argument("out")
    k.add_argument("pmc_csv", nargs="+")
    k.add_argument("--kernel", required=True)
    k.add_argument("--cmd", action="append", default=[])
    a = ap.parse_args(argv)
    if a.mode == "kernel":
        kernel_counters(a.pmc_csv, a.out, a.kernel, a.cmd)
    elif a.mode == "trace":
        trace(a.stats_csv, a.out, a.cmd)
    elif a.mode == "counters":
        counters(a.pmc_csv, a.out, a.cmd, a.simds, a.xcds)
    else:
        traffic(a.fetch_csv, a.write_csv, a.out, a.kernel, a.copy_bytes, a.cmd)


if __name__ == "__main__":
    main()
