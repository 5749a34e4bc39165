#!/usr/bin/env python3
"""Throughput of direct all-pairs softened gravity on one MI355X.

One step = one kick-drift-kick leapfrog step of the whole body set:
nbody_leapfrog_step (kick + drift), the O(N^2) force pass and nbody_kick
(closing half-kick).  The force pass is the pair-symmetric one
(nbody_accel_symmetric, launched as its two phases: the panel-pair kernel,
then the reduce) unless --path tile selects the one-sided nbody_accel.  The
default workload is the N = 1,048,576 Plummer sphere (equal masses 1/N,
eps^2 = 1e-4, dt = 1e-4).  value = N^2 body-body interactions per step /
seconds per step, in billions per second.

Inputs are resident in HBM before the timed region; the region is bracketed by
torch.cuda.synchronize() on both sides.  Every GPU time is taken with the
library's own HIP events (nbody_timer_*, nbody_time_accel), recorded on the
stream the kernels are launched on (the current torch stream); torch only
provides device memory and the stream.  The roofline object reports the
force pass's dominant kernel (the panel-pair kernel, or the one-sided kernel)
against the MI355X FP32 vector peak at 20 flops per interaction (the count of
"Cuda Nbody Notes"); force_ms is the whole pass, the pair-symmetric reduce
kernel included, and force_pass_frac the same ratio for the whole pass.

The energy / momentum pass (a checkpoint diagnostic, not part of a step) is
timed separately.  The CPU baseline is the double-precision oracle timed on a
bounded sample of the same workload's rows on the host cores.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FLOPS_PER_INTERACTION = 20          # "Cuda Nbody Notes", pair-step comments
PEAK_FP32_TFLOPS = 157.3            # MI355X FP32 vector, 256 CU x 64 lanes x 2 x 2 x 2.4 GHz
METRIC = "body-body interactions/s (billions), N=1M fp32; % of MI355X FP32 VALU peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_per_launch(path, variant, workload):
    """HBM bytes per force launch from the committed counter record of this
    force path, variant and workload, or None when there is none or it was
    taken on a different kernel source."""
    from direct_all_pairs_softened_amd.counters import kernel_source_hash, traffic_file
    try:
        with open(traffic_file(path, workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("path"), t.get("variant"), t.get("workload")) != (path, variant, workload):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash(path):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(pm_np, acc0_np, w, seconds):
    """The oracle, untuned, on a bounded sample of rows: each row is the full
    N-term double-precision sum.  Returns the JSON object."""
    import numpy as np
    import oracle
    pos, mass = oracle.split_posmass(pm_np)
    G, eps2 = float(np.float32(w.G)), float(np.float32(w.eps2))
    g = np.random.default_rng(123)
    probe = np.sort(g.choice(w.n, 64, replace=False))
    t0 = time.perf_counter()
    oracle.accel_rows(pos, mass, G, eps2, probe)
    rate = 64 / max(time.perf_counter() - t0, 1e-6)
    rows = int(min(w.n, max(64, rate * seconds)))
    sample = np.sort(g.choice(w.n, rows, replace=False))
    t0 = time.perf_counter()
    ref = oracle.accel_rows(pos, mass, G, eps2, sample)
    dt = time.perf_counter() - t0
    got = acc0_np[sample, :3].astype(np.float64)
    l2 = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    per = float((np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)).max())
    inter = rows * w.n
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")),
                         None)
    except OSError:
        pass
    return {
        "value": inter / dt / 1e9,
        "unit": "billion interactions/s",
        "cores": oracle.num_threads(),
        "cpu_model": model,
        "kind": "oracle",
        "sample": f"{rows} of {w.n} bodies, each summed over all {w.n} (float64, "
                  f"{inter:.3e} interactions in {dt:.1f} s)",
        "sample_parity_vs_gpu": {"rel_l2": l2, "worst_body_rel": per},
    }


SPLITJ_CHUNKS = (32, 256, 1024, 4096, 16384)
# (j_chunk, terms) of the tree first pass: the README's 32-wide block as a
# plain tree, FADL and fadl4, then wider trees
SPLITJ_TREES = ((32, 1), (32, 2), (32, 4), (64, 1), (64, 2), (128, 2), (256, 4))
SPLITJ_MAX_WORKSPACE = 16 << 30


def _time(nb, fn, reps):
    """Milliseconds of each of `reps` calls of fn (after one untimed call),
    between marks of the library's timer on the current stream."""
    fn()
    t = nb.Timer(2 * reps)
    for r in range(reps):
        t.mark(2 * r)
        fn()
        t.mark(2 * r + 1)
    ms = [t.elapsed_ms(2 * r, 2 * r + 1) for r in range(reps)]
    t.close()
    return ms


def _sweep_line(w, ms, **kw):
    inter = float(w.n) * float(w.n)
    best = min(ms)
    tflops = FLOPS_PER_INTERACTION * inter / (best * 1e-3) / 1e12
    print(json.dumps({"workload": w.name, "n": w.n, **kw, "ms_min": best,
                      "ms_avg": sum(ms) / len(ms),
                      "interactions_per_s_billions": inter / (best * 1e-3) / 1e9,
                      "pct_fp32_peak": 100 * tflops / PEAK_FP32_TFLOPS}), flush=True)


def sweep(nb, torch, w, pm, acc, reps, paths):
    """Force-pass time of every compiled variant on the workload, then of the
    two-pass split-j decomposition for a range of chunk widths (workspace
    permitting)."""
    for v in range(nb.nbody_accel_variant_count() if "tile" in paths else 0):
        ms = _time(nb, lambda: nb.nbody_accel_variant(pm, w.G, w.eps2, acc, v), reps)
        _sweep_line(w, ms, variant=v, tiling=nb.nbody_accel_variant_info(v))
    for v in range(nb.nbody_accel_symmetric_variant_count() if "symmetric" in paths else 0):
        need = nb.nbody_accel_symmetric_workspace_bytes(w.n, v)
        if need > 4 * SPLITJ_MAX_WORKSPACE:
            continue
        ws = torch.empty(need, dtype=torch.uint8, device=pm.device)
        ms = _time(nb, lambda: nb.nbody_accel_symmetric(pm, w.G, w.eps2, acc, ws, v), reps)
        _sweep_line(w, ms, symmetric_variant=v, panel=nb.nbody_accel_symmetric_panel(v),
                    workspace_bytes=need)
        del ws
    if "range" in paths:
        # one GPU's share of an i-split over 8 GPUs: N/8 i-bodies against all N
        ni = w.n // 8
        out = torch.empty((ni, 4), dtype=torch.float32, device=pm.device)
        for v in range(nb.nbody_accel_variant_count()):
            ms = _time(nb, lambda: nb.nbody_accel_range(pm, 0, ni, w.G, w.eps2, out, v), reps)
            best = min(ms)
            inter = float(ni) * float(w.n)
            tflops = FLOPS_PER_INTERACTION * inter / (best * 1e-3) / 1e12
            print(json.dumps({"workload": w.name, "n": w.n, "share": [0, ni], "range_variant": v,
                              "tiling": nb.nbody_accel_variant_info(v), "ms_min": best,
                              "interactions_per_s_billions": inter / (best * 1e-3) / 1e9,
                              "pct_fp32_peak": 100 * tflops / PEAK_FP32_TFLOPS}), flush=True)
    for j_chunk in SPLITJ_CHUNKS if "splitj" in paths else ():
        need = nb.nbody_accel_splitj_workspace_bytes(w.n, j_chunk)
        if need > SPLITJ_MAX_WORKSPACE or -(-w.n // j_chunk) > 65535:
            continue
        ws = torch.empty(need, dtype=torch.uint8, device=pm.device)
        ms = _time(nb, lambda: nb.nbody_accel_splitj(pm, w.G, w.eps2, acc, j_chunk, ws), reps)
        _sweep_line(w, ms, splitj_chunk=j_chunk, workspace_bytes=need)
        del ws
    for j_chunk, terms in SPLITJ_TREES if "splitj" in paths else ():
        need = nb.nbody_accel_splitj_tree_workspace_bytes(w.n, j_chunk, terms)
        if need > SPLITJ_MAX_WORKSPACE or -(-w.n // j_chunk) > 65535:
            continue
        ws = torch.empty(need, dtype=torch.uint8, device=pm.device)
        ms = _time(nb, lambda: nb.nbody_accel_splitj_tree(pm, w.G, w.eps2, acc, j_chunk, terms,
                                                             ws), reps)
        _sweep_line(w, ms, splitj_tree_chunk=j_chunk, terms=terms, workspace_bytes=need)
        del ws


# timed force passes per workload in --suite (repetitions per workload)
SUITE_REPS = {"uniform1k": 100, "plummer16k": 100, "lognormal128k": 50, "plummer1m": 10,
              "collision1m": 5}


def _stats(w, ms, interactions=None):
    ms = sorted(ms)
    med = ms[len(ms) // 2] if len(ms) % 2 else 0.5 * (ms[len(ms) // 2 - 1] + ms[len(ms) // 2])
    inter = float(w.n) * float(w.n) if interactions is None else interactions
    return {"reps": len(ms), "ms_median": med, "ms_min": ms[0],
            "interactions_per_s_billions": inter / (med * 1e-3) / 1e9,
            "pct_fp32_peak": 100 * FLOPS_PER_INTERACTION * inter / (med * 1e-3) / 1e12
            / PEAK_FP32_TFLOPS}


def suite(nb, torch, names):
    """One JSON line per workload: force-pass times of the passes that apply
    to it (median and min over the workload's reps), and for workloads with
    dynamics the whole KDK run, timed once, with its energy drift and
    momentum change measured by nbody_energy."""
    import workloads
    dev = torch.device("cuda:0")
    for name in names:
        w = workloads.WORKLOADS[name]
        reps = SUITE_REPS[name]
        log(f"suite {name}: {w.description}")
        pm_np, vel_np = workloads.make(name)
        pm = torch.from_numpy(pm_np).to(dev)
        acc = torch.empty_like(pm)
        out = {"workload": name, "n": w.n, "eps2": w.eps2}
        force = {}
        tv = nb.nbody_accel_variant_for_n(w.n)
        force[f"one_sided_v{tv}"] = _stats(
            w, _time(nb, lambda: nb.nbody_accel_variant(pm, w.G, w.eps2, acc, tv), reps))
        sv = nb.nbody_accel_symmetric_variant_for_n(w.n)
        sym_ws = torch.empty(max(nb.nbody_accel_symmetric_workspace_bytes(w.n, sv), 16),
                             dtype=torch.uint8, device=dev)
        force[f"symmetric_v{sv}"] = _stats(
            w, _time(nb, lambda: nb.nbody_accel_symmetric(pm, w.G, w.eps2, acc, sym_ws, sv),
                     reps))
        if w.n >= 100000:
            pv = nb.nbody_accel_symmetric_potential_variant_for_n(w.n)
            pot_ws = torch.empty(nb.nbody_accel_symmetric_potential_workspace_bytes(w.n, pv),
                                 dtype=torch.uint8, device=dev)
            force[f"symmetric_potential_v{pv}"] = _stats(
                w, _time(nb, lambda: nb.nbody_accel_symmetric_potential(
                    pm, w.G, w.eps2, acc, pot_ws, pv), reps))
            del pot_ws
        if name == "plummer1m":
            # the same one-sided arithmetic over 96-bit float3 records and SoA
            pos3 = pm[:, :3].contiguous()
            mass = pm[:, 3].contiguous()
            acc3 = torch.empty_like(pos3)
            force[f"one_sided_v{tv}_float3_aos"] = _stats(
                w, _time(nb, lambda: nb.nbody_accel_f3aos(pos3, mass, w.G, w.eps2, acc3),
                         reps))
            xyz = [pm[:, k].contiguous() for k in range(4)]
            axyz = [torch.empty_like(xyz[0]) for _ in range(3)]
            force[f"one_sided_v{tv}_soa"] = _stats(
                w, _time(nb, lambda: nb.nbody_accel_soa(*xyz, w.G, w.eps2, *axyz), reps))
            del pos3, mass, acc3, xyz, axyz
        if name == "lognormal128k":
            for j_chunk in SPLITJ_CHUNKS:
                ws = torch.empty(nb.nbody_accel_splitj_workspace_bytes(w.n, j_chunk),
                                 dtype=torch.uint8, device=dev)
                force[f"splitj_J{j_chunk}"] = _stats(
                    w, _time(nb, lambda: nb.nbody_accel_splitj(pm, w.G, w.eps2, acc, j_chunk,
                                                                  ws), reps))
                del ws
            for j_chunk, terms in SPLITJ_TREES:
                ws = torch.empty(nb.nbody_accel_splitj_tree_workspace_bytes(w.n, j_chunk, terms),
                                 dtype=torch.uint8, device=dev)
                force[f"splitj_tree_J{j_chunk}_F{terms}"] = _stats(
                    w, _time(nb, lambda: nb.nbody_accel_splitj_tree(pm, w.G, w.eps2, acc,
                                                                       j_chunk, terms, ws), reps))
                del ws
        out["force"] = force
        if w.steps > 0:
            # the run uses whichever of the two passes was faster here
            best = min(("one_sided", "symmetric"),
                       key=lambda k: next(v["ms_median"] for f, v in force.items()
                                          if f.startswith(k) and "_float3" not in f
                                          and "_soa" not in f))
            if best == "symmetric":
                def fpass():
                    nb.nbody_accel_symmetric(pm, w.G, w.eps2, acc, sym_ws, sv)
            else:
                def fpass():
                    nb.nbody_accel_variant(pm, w.G, w.eps2, acc, tv)
            vel = torch.from_numpy(vel_np).to(dev)
            e0 = nb.energy(pm, vel, w.G, w.eps2)
            fpass()
            timer = nb.Timer(w.steps + 1)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            timer.mark(0)
            for k in range(w.steps):
                nb.nbody_leapfrog_step(pm, vel, acc, w.dt)
                fpass()
                nb.nbody_kick(vel, acc, 0.5 * w.dt)
                timer.mark(k + 1)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            step_ms = [timer.elapsed_ms(k, k + 1) for k in range(w.steps)]
            timer.close()
            e1 = nb.energy(pm, vel, w.G, w.eps2)
            dp = sum((e1[c] - e0[c]) ** 2 for c in ("Px", "Py", "Pz")) ** 0.5
            out["run"] = {"steps": w.steps, "dt": w.dt, "force_pass": best,
                          "wall_s": wall, "step_ms_median": sorted(step_ms)[len(step_ms) // 2],
                          "E0": e0["E"], "E1": e1["E"],
                          "energy_drift": abs(e1["E"] - e0["E"]) / abs(e0["E"]),
                          "momentum_change": dp}
            del vel
        if w.n <= 20000:
            # launch-bound sizes: the library's step loop, eager and as a HIP graph
            fastest = min(("one_sided", "symmetric"),
                          key=lambda k: next(v["ms_median"] for f, v in force.items()
                                             if f.startswith(k)))
            out["kdk_run"] = kdk_run_timing(nb, torch, w, pm_np, vel_np, fastest, sym_ws, sv,
                                            tv)
        if name == "plummer1m":
            vel = torch.from_numpy(vel_np).to(dev)
            sv_ws = sym_ws

            def kdk():
                nb.nbody_leapfrog_step(pm, vel, acc, w.dt)
                nb.nbody_accel_symmetric(pm, w.G, w.eps2, acc, sv_ws, sv)
                nb.nbody_kick(vel, acc, 0.5 * w.dt)
            nb.nbody_accel_symmetric(pm, w.G, w.eps2, acc, sym_ws, sv)
            out["kdk_step"] = _stats(w, _time(nb, kdk, 3))
            del vel
        print(json.dumps(out), flush=True)
        del pm, acc, sym_ws
        torch.cuda.empty_cache()


def kdk_run_timing(nb, torch, w, pm_np, vel_np, best, sym_ws, sv, tv, steps=200):
    """`steps` kick-drift-kick steps from the workload's initial state, run by
    the library's loop (nbody_kdk_run) and as the calls made one by one
    (nbody_leapfrog_step, the force pass, nbody_kick): ms per step between
    events around the whole run.  The two final states must be bitwise
    equal."""
    dev = torch.device("cuda:0")
    dt = w.dt if w.dt > 0 else 1e-3   # a workload without dynamics of its own
    sym = best == "symmetric"
    kind = nb.NBODY_PASS_SYMMETRIC if sym else nb.NBODY_PASS_ONE_SIDED
    variant = sv if sym else tv
    ws = sym_ws if sym else None

    def fpass(pm, acc):
        if sym:
            nb.nbody_accel_symmetric(pm, w.G, w.eps2, acc, ws, variant)
        else:
            nb.nbody_accel_variant(pm, w.G, w.eps2, acc, variant)

    res, finals = {}, {}
    # untimed: the first steps after a change of work run slow (clocks, caches)
    pm = torch.from_numpy(pm_np).to(dev)
    vel = torch.from_numpy(vel_np).to(dev)
    acc = torch.empty_like(pm)
    fpass(pm, acc)
    nb.nbody_kdk_run(pm, vel, acc, w.G, w.eps2, dt, steps // 4, kind, variant, ws)
    torch.cuda.synchronize()
    for how in ("library", "calls"):
        pm = torch.from_numpy(pm_np).to(dev)
        vel = torch.from_numpy(vel_np).to(dev)
        acc = torch.empty_like(pm)
        fpass(pm, acc)
        torch.cuda.synchronize()
        t = nb.Timer(2)
        t.mark(0)
        if how == "library":
            nb.nbody_kdk_run(pm, vel, acc, w.G, w.eps2, dt, steps, kind, variant, ws)
        else:
            for _ in range(steps):
                nb.nbody_leapfrog_step(pm, vel, acc, dt)
                fpass(pm, acc)
                nb.nbody_kick(vel, acc, 0.5 * dt)
        t.mark(1)
        res[how] = t.elapsed_ms(0, 1) / steps
        t.close()
        finals[how] = [x.cpu() for x in (pm, vel, acc)]
    same = all(torch.equal(a, b) for a, b in zip(finals["library"], finals["calls"]))
    if not same:
        raise AssertionError("nbody_kdk_run differs from the calls made one by one")
    return {"steps": steps, "force_pass": best, "library_ms_per_step": res["library"],
            "calls_ms_per_step": res["calls"], "bitwise_equal": same}


def suite_report(path):
    """Markdown tables of the JSON lines written by --suite (formatting only)."""
    recs = [json.loads(line) for line in open(path) if line.strip().startswith("{")]
    out = ["| workload | pass | reps | median ms | min ms | 10^9 interactions/s | % of 157.3 TF |",
           "|---|---|---|---|---|---|---|"]
    for r in recs:
        for name, f in r["force"].items():
            out.append("| %s | %s | %d | %.4g | %.4g | %.0f | %.1f |" % (
                r["workload"], name, f["reps"], f["ms_median"], f["ms_min"],
                f["interactions_per_s_billions"], f["pct_fp32_peak"]))
    out += ["", "| workload | steps x dt | force pass | median step ms | energy drift | "
            "momentum change |", "|---|---|---|---|---|---|"]
    for r in recs:
        run = r.get("run")
        if run:
            out.append("| %s | %d x %g | %s | %.4g | %.2e | %.2e |" % (
                r["workload"], run["steps"], run["dt"], run["force_pass"],
                run["step_ms_median"], run["energy_drift"], run["momentum_change"]))
    runs = [r for r in recs if r.get("kdk_run")]
    if runs:
        out += ["", "| workload | steps | force pass | nbody_kdk_run ms per step | "
                "calls one by one ms per step | bitwise equal |", "|---|---|---|---|---|---|"]
        for r in runs:
            k = r["kdk_run"]
            out.append("| %s | %d | %s | %.4g | %.4g | %s |" % (
                r["workload"], k["steps"], k["force_pass"], k["library_ms_per_step"],
                k["calls_ms_per_step"], "yes" if k["bitwise_equal"] else "no"))
    print("\n".join(out))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="plummer1m")
    ap.add_argument("--path", choices=("tile", "symmetric", "symmetric_chunked"),
                    default="symmetric",
                    help="force pass: one-sided LDS-tiled (nbody_accel), pair-symmetric "
                         "(nbody_accel_symmetric), or pair-symmetric in column chunks "
                         "(nbody_accel_symmetric_chunked)")
    ap.add_argument("--chunk", type=int, default=0,
                    help="panels per chunk for --path symmetric_chunked (0: the library's)")
    ap.add_argument("--variant", type=int, default=None, help="force a compiled force variant")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target length of the oracle CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-one-sided", action="store_true",
                    help="skip timing the one-sided pass beside the pair-symmetric one")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip timing the chunked pair-symmetric pass beside the whole one")
    ap.add_argument("--sweep", action="store_true",
                    help="time the force pass of every compiled variant (one JSON line each) "
                         "instead of the step benchmark")
    ap.add_argument("--reps", type=int, default=3, help="timed force passes per variant (--sweep)")
    ap.add_argument("--suite", default=None, metavar="NAMES",
                    help="comma-separated workloads (or 'all'): per-workload force-pass times "
                         "and whole KDK runs, one JSON line each, instead of the step benchmark")
    ap.add_argument("--sweep-paths", default="tile,symmetric,splitj",
                    help="comma-separated subset of tile, symmetric, splitj, range (--sweep)")
    ap.add_argument("--suite-report", default=None, metavar="JSONL",
                    help="print Markdown tables of a file of --suite output and exit (no GPU)")
    args = ap.parse_args()
    if args.suite_report:
        suite_report(args.suite_report)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(the force pass would shard by i with an all-gather of positions).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import direct_all_pairs_softened_amd as nb
    import workloads

    nb.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.suite:
        names = (list(workloads.WORKLOADS) if args.suite == "all"
                 else args.suite.split(","))
        suite(nb, torch, names)
        return
    w = workloads.WORKLOADS[args.workload]
    dt = w.dt if w.dt > 0 else 1e-4
    log(f"workload {w.name}: {w.description}")
    pm_np, vel_np = workloads.make(w.name)
    dev = torch.device("cuda:0")
    pm = torch.from_numpy(pm_np).to(dev)
    vel = torch.from_numpy(vel_np).to(dev)
    acc = torch.empty_like(pm)
    if args.sweep:
        sweep(nb, torch, w, pm, acc, args.reps, set(args.sweep_paths.split(",")))
        return
    if args.path == "symmetric":
        variant = (args.variant if args.variant is not None
                   else nb.nbody_accel_symmetric_variant_for_n(w.n))
        ws_bytes = nb.nbody_accel_symmetric_workspace_bytes(w.n, variant)
        sym_ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        info = {"path": "symmetric", "panel": nb.nbody_accel_symmetric_panel(variant),
                "workspace_bytes": ws_bytes}

        # the pass in its two phases (the same kernels as one
        # nbody_accel_symmetric call), so that events can bracket the
        # panel-pair kernel, the dominant one, on its own
        def force_main():
            nb.nbody_accel_symmetric_tasks(pm, w.eps2, sym_ws, variant)

        def force_rest():
            nb.nbody_accel_symmetric_reduce(w.n, w.G, acc, sym_ws, variant)
    elif args.path == "symmetric_chunked":
        variant = (args.variant if args.variant is not None
                   else nb.nbody_accel_symmetric_variant_for_n(w.n))
        ws_bytes = nb.nbody_accel_symmetric_chunked_workspace_bytes(w.n, variant, args.chunk)
        sym_ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        info = {"path": "symmetric_chunked", "panel": nb.nbody_accel_symmetric_panel(variant),
                "chunk_panels": args.chunk or 32, "workspace_bytes": ws_bytes}

        # every chunk's panel-pair and reduce kernels: the events bracket the
        # whole pass
        def force_main():
            nb.nbody_accel_symmetric_chunked(pm, w.G, w.eps2, acc, sym_ws, variant, args.chunk)

        def force_rest():
            pass
    else:
        variant = args.variant if args.variant is not None else nb.nbody_accel_variant_for_n(w.n)
        info = dict(nb.nbody_accel_variant_info(variant), path="tile")

        def force_main():
            nb.nbody_accel_variant(pm, w.G, w.eps2, acc, variant)

        def force_rest():
            pass

    def force():
        force_main()
        force_rest()

    force()
    torch.cuda.synchronize()
    acc0_np = acc.cpu().numpy()

    def step():
        nb.nbody_leapfrog_step(pm, vel, acc, dt)
        force()
        nb.nbody_kick(vel, acc, 0.5 * dt)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # marks: 0 at the start, then per step k: after the kick-drift (4k + 1),
    # after the dominant kernel (4k + 2), after the force pass (4k + 3) and
    # after the closing half-kick (4k + 4)
    timer = nb.Timer(4 * args.steps + 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    timer.mark(0)
    for k in range(args.steps):
        nb.nbody_leapfrog_step(pm, vel, acc, dt)
        timer.mark(4 * k + 1)
        force_main()
        timer.mark(4 * k + 2)
        force_rest()
        timer.mark(4 * k + 3)
        nb.nbody_kick(vel, acc, 0.5 * dt)
        timer.mark(4 * k + 4)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kernel_ms = [timer.elapsed_ms(4 * k + 1, 4 * k + 2) for k in range(args.steps)]
    force_ms = [timer.elapsed_ms(4 * k + 1, 4 * k + 3) for k in range(args.steps)]
    step_ms = [timer.elapsed_ms(4 * k, 4 * k + 4) for k in range(args.steps)]
    timer.close()
    kernel_avg = sum(kernel_ms) / len(kernel_ms)
    force_avg = sum(force_ms) / len(force_ms)
    inter = float(w.n) * float(w.n)
    value = inter / (ms_per_step * 1e-3) / 1e9
    achieved = FLOPS_PER_INTERACTION * inter / (kernel_avg * 1e-3) / 1e12
    pass_tflops = FLOPS_PER_INTERACTION * inter / (force_avg * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms (events {sum(step_ms) / len(step_ms):.3f}), force pass "
        f"{force_avg:.3f} ms, its main kernel {kernel_avg:.3f} ms (min {min(kernel_ms):.3f}), "
        f"{value:.1f} G interactions/s per step")

    # the one-sided pass (nbody_accel, no workspace) on the same positions, for
    # comparison
    one_ms = None
    if args.path != "tile" and not args.no_one_sided:
        one_ms, _ = nb.nbody_time_accel(pm, w.G, w.eps2, acc, nb.NBODY_PASS_ONE_SIDED, 2)
        log(f"one-sided nbody_accel: {min(one_ms):.3f} ms")

    # the same pass in column chunks (bounded workspace, bitwise equal)
    chunked_ms = chunked_ws = None
    if args.path == "symmetric" and not args.no_chunked:
        chunked_ws = nb.nbody_accel_symmetric_chunked_workspace_bytes(w.n, variant)
        cws = torch.empty(chunked_ws, dtype=torch.uint8, device=dev)
        chunked_ms = min(_time(nb, lambda: nb.nbody_accel_symmetric_chunked(
            pm, w.G, w.eps2, acc, cws, variant), 2))
        del cws
        log(f"chunked pass: {chunked_ms:.3f} ms in {chunked_ws / 2**30:.2f} GiB")

    # energy diagnostic (outside the timed steps)
    ws = torch.empty(nb.nbody_energy_workspace_bytes(w.n), dtype=torch.uint8, device=dev)
    stats = torch.zeros(8, dtype=torch.float64, device=dev)
    energy_ms = _time(nb, lambda: nb.nbody_energy(pm, vel, w.G, w.eps2, ws, stats), 1)[0]
    checkpoint_ms = None
    if args.path != "tile":
        # a checkpoint step's force pass with the potentials in accel.w, then
        # the O(N) energy from them (in place of force pass + energy pass)
        pv = nb.nbody_accel_symmetric_potential_variant_for_n(w.n)
        pot_ws = torch.empty(nb.nbody_accel_symmetric_potential_workspace_bytes(w.n, pv),
                             dtype=torch.uint8, device=dev)
        pws = torch.empty(nb.nbody_energy_from_potential_workspace_bytes(w.n),
                          dtype=torch.uint8, device=dev)
        acc_pot = torch.empty_like(acc)

        def checkpoint():
            nb.nbody_accel_symmetric_potential(pm, w.G, w.eps2, acc_pot, pot_ws, pv)
            nb.nbody_energy_from_potential(pm, vel, acc_pot, pws, stats)
        checkpoint_ms = _time(nb, checkpoint, 1)[0]
        del pot_ws, pws, acc_pot

    # FP32 arithmetic the pair step actually issues (rsq not counted), per
    # counted interaction: the pair-symmetric step evaluates each pair once
    # for two interactions (3 sub, 1 fma, 2 fmac, 4 mul, 6 fmac = 25 flops),
    # the one-sided step 3 sub, 3 fma, 3 mul, 3 fmac = 18 flops
    issued = 18.0 if args.path == "tile" else 12.5
    traffic = traffic_per_launch(args.path, variant, w.name)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "billion interactions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "n": w.n,
            "bodies": w.description,
            "eps2": w.eps2,
            "G": w.G,
            "dt": dt,
            "step": "kick+drift, force pass, half-kick",
            "force_variant": variant,
            "force_tiling": info,
        },
        "pct_fp32_peak": 100.0 * achieved / PEAK_FP32_TFLOPS,
        "force_ms": force_avg,
        "force_kernel_ms": kernel_avg,
        "force_pass_frac": pass_tflops / PEAK_FP32_TFLOPS,
        "pairs_evaluated_per_interaction": 1.0 if args.path == "tile" else 0.5,
        "fp32_flops_issued_per_interaction": issued,
        "fp32_issued_frac": issued * inter / (kernel_avg * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
        "chunked_force_ms": chunked_ms,
        "chunked_workspace_bytes": chunked_ws,
        "one_sided_force_ms": min(one_ms) if one_ms else None,
        "one_sided_frac": (FLOPS_PER_INTERACTION * inter / (min(one_ms) * 1e-3) / 1e12
                           / PEAK_FP32_TFLOPS) if one_ms else None,
        "energy_ms": energy_ms,
        "checkpoint_force_energy_ms": checkpoint_ms,
        "roofline": {
            "bound": "alu",
            "achieved": achieved,
            "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_TFLOPS,
            "traffic": traffic,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the oracle on a row sample ...")
        out["cpu_baseline"] = cpu_baseline(pm_np, acc0_np, w, args.cpu_seconds)
        log(f"cpu baseline: {out['cpu_baseline']['value']:.3f} G interactions/s on "
            f"{out['cpu_baseline']['cores']} threads")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
