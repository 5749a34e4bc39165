"""Hardware-counter runs of the force pass (run under rocprofv3 --pmc).

``run``: one calibration copy of a known number of bytes (torch's copy
kernel, HBM to HBM), then one force pass of a workload.  Profile it once per
counter group, e.g.

    rocprofv3 --pmc FETCH_SIZE -d DIR/fetch -o run -- \\
        python3 -m direct_all_pairs_softened_amd.counters run --workload plummer1m

``summarize``: reads the counter_collection CSVs of those runs and writes a
JSON record (HBM bytes per force launch, scaled by what the same counters
read for the copy) and a Markdown table.

FETCH_SIZE and WRITE_SIZE are in KiB per dispatch; each is scaled by
copy_bytes / (counter reading of the copy), so a counter that over- or
under-counts by a constant factor is corrected.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 30
# the force kernel whose counters a record holds, per force path
FORCE_KERNELS = {"symmetric": ("symmetric_task_kernel",), "tile": ("force_tile_kernel",)}
# the sources that kernel is built from: a record is valid for a build only
# while their hash matches
KERNEL_SOURCES = {
    "symmetric": ("direct_all_pairs_softened_amd/csrc/symmetric.hip",
                  "direct_all_pairs_softened_amd/csrc/nbody_common.hpp"),
    "tile": ("direct_all_pairs_softened_amd/csrc/force.hip",
             "direct_all_pairs_softened_amd/csrc/nbody_common.hpp"),
}
COPY_KERNEL_HINTS = ("copyBuffer", "copy", "Copy")


def _code_only(text: str) -> str:
    """C++ source without comments, whitespace runs collapsed: edits to
    comments or layout do not count as a change of the kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(path: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[path]:
        with open(os.path.join(ROOT, rel)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def cmd_run(args):
    sys.path.insert(0, ROOT)
    import torch

    import direct_all_pairs_softened_amd as nb
    import workloads

    w = workloads.WORKLOADS[args.workload]
    pm_np, _ = workloads.make(w.name)
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)          # device-to-device copy of COPY_BYTES
    torch.cuda.synchronize()
    pm = torch.from_numpy(pm_np).to(dev)
    acc = torch.empty_like(pm)
    if args.path == "energy":
        vel = torch.from_numpy(workloads.make(w.name)[1]).to(dev)
        ws = torch.empty(nb.nbody_energy_workspace_bytes(w.n), dtype=torch.uint8, device=dev)
        stats = torch.zeros(8, dtype=torch.float64, device=dev)
        nb.nbody_energy(pm, vel, w.G, w.eps2, ws, stats)
        torch.cuda.synchronize()
        print(f"counters run: copy {COPY_BYTES} B, energy on {w.name}", flush=True)
        return
    if args.path == "symmetric":
        v = args.variant if args.variant is not None else nb.nbody_accel_symmetric_variant_for_n(w.n)
        ws = torch.empty(nb.nbody_accel_symmetric_workspace_bytes(w.n, v), dtype=torch.uint8,
                         device=dev)
        for _ in range(args.reps):
            nb.nbody_accel_symmetric(pm, w.G, w.eps2, acc, ws, v)
    elif args.path == "symmetric_chunked":
        v = args.variant if args.variant is not None else nb.nbody_accel_symmetric_variant_for_n(w.n)
        ws = torch.empty(nb.nbody_accel_symmetric_chunked_workspace_bytes(w.n, v),
                         dtype=torch.uint8, device=dev)
        for _ in range(args.reps):
            nb.nbody_accel_symmetric_chunked(pm, w.G, w.eps2, acc, ws, v)
    else:
        v = args.variant if args.variant is not None else nb.nbody_accel_variant_for_n(w.n)
        for _ in range(args.reps):
            nb.nbody_accel_variant(pm, w.G, w.eps2, acc, v)
    torch.cuda.synchronize()
    print(f"counters run: copy {COPY_BYTES} B, {args.path} force variant {v} on {w.name}",
          flush=True)


def cmd_sq_report(args):
    """Prints the SQ/GRBM counters of the first dispatch of a kernel and the
    rates derived from them (MI355X: 8 XCDs, 256 CUs, 4 SIMDs per CU)."""
    c = read_counters(os.path.join(args.dir, "**", "*counter_collection.csv"))
    name, v = pick(c, (args.kernel,))
    print(f"kernel: `{name}`")
    print("")
    print("| counter | value |")
    print("|---|---|")
    for k in sorted(v):
        print(f"| {k} | {v[k]:.4e} |")
    print("")
    g = v.get("GRBM_GUI_ACTIVE", 0.0) / 8
    if g:
        print(f"- cycles per XCD (GRBM_GUI_ACTIVE / 8): {g:.4e}")
        if args.ms:
            print(f"- clock over {args.ms:.2f} ms: {g / (args.ms * 1e-3) / 1e9:.2f} GHz")
        if "SQ_INSTS_VALU" in v:
            print(f"- VALU instructions per SIMD quad-cycle: {v['SQ_INSTS_VALU'] / 1024 / (g / 4):.3f}")
        if "SQ_ACTIVE_INST_VALU2" in v:
            print(f"- quad-cycles issuing two VALU instructions: "
                  f"{100 * v['SQ_ACTIVE_INST_VALU2'] / (g * 256):.1f} %")
        if "SQ_BUSY_CU_CYCLES" in v:
            print(f"- SIMD quad-cycles busy: {100 * v['SQ_BUSY_CU_CYCLES'] / (g * 256):.1f} %")
        if "SQ_WAVE_CYCLES" in v:
            # SQ_WAVE_CYCLES adds the resident waves every fourth cycle
            print(f"- mean resident waves per SIMD: {4 * v['SQ_WAVE_CYCLES'] / g / 1024:.2f}")


def read_counters(pattern):
    """{(dispatch_id, kernel_name): {counter: summed value}} from counter CSVs."""
    out = defaultdict(lambda: defaultdict(float))
    files = glob.glob(pattern, recursive=True)
    if not files:
        raise FileNotFoundError(pattern)
    for path in files:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                key = (int(row["Dispatch_Id"]), row["Kernel_Name"])
                out[key][row["Counter_Name"]] += float(row["Counter_Value"])
    return out


def pick(rows, hint_list):
    for (did, name), vals in sorted(rows.items()):
        if any(h in name for h in hint_list):
            return name, vals
    raise KeyError(f"no kernel matching {hint_list}")


def algorithmic_bytes(kernel_name: str, n: int, panel: int) -> int:
    """One-sided pass: 16 B read + 16 B written per body.  Pair-symmetric task
    kernel: 16 B read per body plus its P^2 panel sums of 3 floats per body
    (12 n P bytes, P = ceil(n / panel)), which the reduce kernel reads back."""
    if "symmetric_task_kernel" in kernel_name:
        P = -(-n // panel)
        return 16 * n + 12 * P * P * panel
    return 32 * n


def traffic_file(path: str, workload: str) -> str:
    """Where the counter record of a force path on a workload is kept."""
    prefix = "force" if path == "symmetric" else "force_tile"
    return os.path.join(ROOT, "profiles", f"{prefix}_{workload}_traffic.json")


def cmd_summarize(args):
    kernels = FORCE_KERNELS[args.path]
    fetch = read_counters(os.path.join(args.fetch_dir, "**", "*counter_collection.csv"))
    write = read_counters(os.path.join(args.write_dir, "**", "*counter_collection.csv"))
    copy_name, cf = pick(fetch, COPY_KERNEL_HINTS)
    kname, ff = pick(fetch, kernels)
    _, cw = pick(write, COPY_KERNEL_HINTS)
    _, fw = pick(write, kernels)
    fetch_scale = COPY_BYTES / (cf["FETCH_SIZE"] * 1024.0)
    write_scale = COPY_BYTES / (cw["WRITE_SIZE"] * 1024.0)
    force_fetch = ff["FETCH_SIZE"] * 1024.0 * fetch_scale
    force_write = fw["WRITE_SIZE"] * 1024.0 * write_scale
    rec = {
        "workload": args.workload,
        "n": args.n,
        "path": args.path,
        "variant": args.variant,
        "kernel": kname,
        "kernel_source_hash": kernel_source_hash(args.path),
        "copy_kernel": copy_name,
        "copy_bytes": COPY_BYTES,
        "copy_fetch_kib": cf["FETCH_SIZE"],
        "copy_write_kib": cw["WRITE_SIZE"],
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "force_fetch_kib": ff["FETCH_SIZE"],
        "force_write_kib": fw["WRITE_SIZE"],
        "hbm_bytes_per_launch": force_fetch + force_write,
        "algorithmic_bytes_per_launch": algorithmic_bytes(kname, args.n, args.panel),
    }
    if args.sq_dir:
        sq = read_counters(os.path.join(args.sq_dir, "**", "*counter_collection.csv"))
        _, fs = pick(sq, kernels)
        rec["sq"] = dict(fs)
    if args.dram_dir:
        dr = read_counters(os.path.join(args.dram_dir, "**", "*counter_collection.csv"))
        _, fd = pick(dr, kernels)
        _, cd = pick(dr, COPY_KERNEL_HINTS)
        rec["tcc"] = {"force": dict(fd), "copy": dict(cd)}
    out_json = args.out_json or traffic_file(args.path, args.workload)
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec, indent=1, sort_keys=True))


def cmd_trace_report(args):
    """Markdown table of a rocprofv3 --stats kernel_stats.csv."""
    files = glob.glob(os.path.join(args.dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(args.dir)
    lines = ["| kernel | calls | avg ms | min ms | max ms | % time |",
             "|---|---|---|---|---|---|"]
    with open(files[0], newline="") as f:
        for row in csv.DictReader(f):
            name = row["Name"]
            if len(name) > 90:
                name = name[:87] + "..."
            lines.append("| `%s` | %s | %.4f | %.4f | %.4f | %.2f |" % (
                name, row["Calls"], float(row["AverageNs"]) / 1e6,
                float(row["MinNs"]) / 1e6, float(row["MaxNs"]) / 1e6,
                float(row["Percentage"])))
    print("\n".join(lines))


def _short_kernel_name(name: str) -> str:
    """Kernel name without namespaces and argument list, template arguments
    kept: symmetric_task_kernel<8, 1, 4, 6, 1>."""
    base = name.replace("(anonymous namespace)::", "").split("(")[0]
    if base.startswith("void "):
        base = base[5:]
    head, sep, tmpl = base.partition("<")
    return head.split("::")[-1] + (sep + tmpl if sep else "")


def cmd_dispatch_report(args):
    """Markdown table of a rocprofv3 kernel_trace.csv with one row per kernel
    and launch shape (grid, block): dispatch count and mean / min duration.
    The same kernel launched on different problem sizes gets separate rows."""
    files = glob.glob(os.path.join(args.dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(args.dir)
    groups = defaultdict(list)
    order = []
    with open(files[0], newline="") as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    prev = ""
    for row in rows:
        name = _short_kernel_name(row["Kernel_Name"])
        key = (name, int(row["Grid_Size_X"]), int(row["Grid_Size_Y"]),
               int(row["Workgroup_Size_X"]), prev if args.by_predecessor else "")
        if key not in groups:
            order.append(key)
        groups[key].append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e6)
        prev = "%s [grid y %s]" % (name.split("<")[0], row["Grid_Size_Y"])
    head = "| kernel | grid x (threads) | grid y | block | dispatches | mean ms | median ms | min ms |"
    rule = "|---|---|---|---|---|---|---|---|"
    if args.by_predecessor:
        head, rule = head + " launched after |", rule + "---|"
    lines = [head, rule]
    for key in order:
        ms = sorted(groups[key])
        if sum(ms) < args.min_total_ms:
            continue
        line = "| `%s` | %d | %d | %d | %d | %.4f | %.4f | %.4f |" % (
            key[0], key[1], key[2], key[3], len(ms), sum(ms) / len(ms), ms[len(ms) // 2], ms[0])
        if args.by_predecessor:
            line += " %s |" % key[4]
        lines.append(line)
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", default="plummer1m")
    r.add_argument("--variant", type=int, default=None)
    r.add_argument("--reps", type=int, default=1, help="force passes, back to back")
    r.add_argument("--path", choices=("tile", "symmetric", "symmetric_chunked", "energy"),
                   default="symmetric")
    q = sub.add_parser("sq-report", help="SQ/GRBM counters of one kernel, with derived rates")
    q.add_argument("--dir", required=True)
    q.add_argument("--kernel", required=True, help="a substring of the kernel name")
    q.add_argument("--ms", type=float, default=None,
                   help="the kernel's traced duration, for the clock estimate")
    s = sub.add_parser("summarize")
    s.add_argument("--fetch-dir", required=True)
    s.add_argument("--write-dir", required=True)
    s.add_argument("--sq-dir", default=None)
    s.add_argument("--dram-dir", default=None)
    s.add_argument("--path", choices=("tile", "symmetric"), default="symmetric")
    s.add_argument("--variant", type=int, required=True,
                   help="the variant the profiled run used (printed by run)")
    s.add_argument("--workload", default="plummer1m")
    s.add_argument("--n", type=int, default=1 << 20)
    s.add_argument("--panel", type=int, default=2048)
    s.add_argument("--out-json", default=None,
                   help="default: the record bench.py reads for this path and workload")
    t = sub.add_parser("trace-report")
    t.add_argument("--dir", required=True)
    d = sub.add_parser("dispatch-report")
    d.add_argument("--dir", required=True)
    d.add_argument("--min-total-ms", type=float, default=0.0,
                   help="leave out (kernel, shape) groups whose total time is below this")
    d.add_argument("--by-predecessor", action="store_true",
                   help="also split groups by the kernel dispatched just before (tells apart "
                        "second passes that follow first passes of different shapes)")
    a = ap.parse_args()
    {"run": cmd_run, "summarize": cmd_summarize, "trace-report": cmd_trace_report,
     "sq-report": cmd_sq_report,
     "dispatch-report": cmd_dispatch_report}[a.cmd](a)


if __name__ == "__main__":
    main()
