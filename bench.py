#!/usr/bin/env python3
"""Benchmark of the PCG + factorised-SPAI hot path on one MI355X.

Workload: 3D Poisson 7-point Laplacian on a 128^3 interior grid (n = 2,097,152,
nnz = 14,581,760), fp64 CSR, b ~ N(0,1), G on tril(A) with seeded random
values, eps = 3e-3, rtol = 1e-10, adjoint loss L = <w, x> with w ~ N(0,1).

One step = the whole hot path on that input, already resident in HBM:
handle set-up (row binning of A and G, explicit G^T built on the device),
the forward PCG solve, and the adjoint solve with dL/db and dL/dA.
value = PCG iterations (forward + adjoint) per second over the timed steps.

Also reported: the live HIP-event duration of the dominant kernel (the fused
A-product step) and its algorithmic-byte rate against the 8 TB/s HBM peak,
the whole-iteration byte rate, a standalone SpMV rate, and the CPU oracle
timed on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "PCG iters/sec + SpMV HBM GB/s (% of peak), 3D Poisson 128^3 fp64, 1 GPU"
PROF_EVERY = 23
KERNEL_SRCS = [os.path.join(ROOT, "preconditioned_cg_solver_amd", "csrc", f)
               for f in ("solver.hip", "multi.hip", "device_util.h")]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_bytes(A, G, sv, si=4):
    """Bytes the method must move (each matrix stream once, each vector once
    per kernel, gathers counted once), per SpMV and per fused kernel; CSR
    counts (sv + si) bytes per nonzero, 3x3 BSR (9 sv + si) per block."""
    n = A.n

    def spmv(M):
        per = (sv + si) * M.nnz if M.block_dim == 1 else (9 * sv + si) * M.nnzb
        return per + si * (M.n_block_rows + 1) + 2 * sv * n
    a_step = spmv(A) + 3 * sv * n + 3 * sv * n          # SpMV(A) + p update + x update
    gt_step = spmv(G) + 3 * sv * n                      # SpMV(G^T) + r update
    g_step = spmv(G) + sv * n                           # SpMV(G) + eps r
    return {"spmv_A": spmv(A), "a_step": a_step, "gt_step": gt_step, "g_step": g_step,
            "iteration": a_step + gt_step + g_step}


def fused_iteration(A):
    """Whether the library runs the fused iteration on A (p and r formed inside
    the products' gathers): CSR matrices in the SELL-64 layout, unless
    SLA_FUSION overrides.  Otherwise the A kernel is the bare product q = A p
    (with p.q) and the p, x and r updates run as separate streaming passes."""
    e = os.environ.get("SLA_FUSION")
    if e in ("fused", "unfused"):
        return e == "fused"
    return A.block_dim == 1 and sell_layout(A)


def sell_slots(M):
    """Slots of the SELL-64 copy the library builds for short-row CSR (each
    64-row slice padded to its longest row)."""
    import numpy as np
    lens = np.diff(M.row_ptr.astype(np.int64))
    ns = (M.n + 63) // 64
    w = np.zeros(ns, np.int64)
    np.maximum.at(w, np.arange(M.n) // 64, lens)
    return int(w.sum() * 64), ns


def sell_layout(A):
    """Whether the library keeps a CSR matrix in the SELL-64 layout: rows of at
    most 32 entries, slices padded by at most 25 %."""
    import numpy as np
    lens = np.diff(A.row_ptr.astype(np.int64))
    if A.nnz == 0 or lens.max(initial=0) > 32:
        return False
    slots, _ = sell_slots(A)
    return slots * 100 <= A.nnz * 125


def slice_offset_slots(M):
    """Slots of the library's slice-offset form of SELL-64 (every 64-row slice
    lists the distinct column offsets of its rows, at most 8, and slot j holds
    offset j for each row), or None when the rows do not qualify: a row with
    unsorted columns, a slice with more than 8 offsets, padding above 25 %, or
    SLA_SELL_OFS=0."""
    import numpy as np
    if os.environ.get("SLA_SELL_OFS", "") == "0" or M.nnz == 0:
        return None
    lens = np.diff(M.row_ptr.astype(np.int64))
    rows = np.repeat(np.arange(M.n), lens)
    ci = M.col_idx.astype(np.int64)
    d = ci - rows
    if np.abs(d).max(initial=0) > 32767:
        return None
    same_row = rows[1:] == rows[:-1]
    if np.any(ci[1:][same_row] <= ci[:-1][same_row]):
        return None
    per_slice = np.bincount(np.unique((rows // 64) * 65536 + (d + 32768)) // 65536,
                            minlength=(M.n + 63) // 64)
    if per_slice.max(initial=0) > 8:
        return None
    slots = int(per_slice.sum() * 64)
    return (slots, len(per_slice)) if slots * 100 <= M.nnz * 125 else None


def moved_bytes_a_step(A, n, sv=8):
    """Bytes the fused A step physically streams with the SELL-64 layout:
    values + column words (16-bit offsets where every |col - row| fits; in the
    slice-offset form one 4-byte offset per slot of a slice and a one-byte
    mask per row instead) + slice starts, z, p_old and x read, x, p_new and q
    written (gathers counted once); None for matrices outside that layout."""
    import numpy as np
    if A.block_dim != 1:
        return None
    lens = np.diff(A.row_ptr.astype(np.int64))
    if lens.max(initial=0) > 32:
        return None
    ofs = slice_offset_slots(A)
    if ofs is not None:
        slots, ns = ofs
        return slots * sv + (slots // 64) * 4 + ns * 64 + 4 * (ns + 1) + 6 * sv * n
    rows = np.repeat(np.arange(A.n), lens)
    col_bytes = 2 if np.abs(A.col_idx.astype(np.int64) - rows).max(initial=0) <= 32767 else 4
    slots, ns = sell_slots(A)
    return slots * (sv + col_bytes) + 4 * (ns + 1) + 6 * sv * n


def kernel_source_shas() -> dict:
    """SHA-256 of each source of the counted kernels: the counters of a kernel
    are used only while its own source file and the shared device helpers
    are unchanged."""
    return {os.path.basename(f): hashlib.sha256(open(f, "rb").read()).hexdigest()
            for f in KERNEL_SRCS}


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def traffic_if_current(workload: str):
    """Per-kernel HBM bytes per launch of a workload from the committed
    rocprofv3 counter runs, keeping only the kernels whose sources are
    unchanged since the counters were taken; None if there are none."""
    try:
        rec = json.load(open(traffic_file(workload)))
    except (OSError, ValueError):
        return None
    now, then = kernel_source_shas(), rec.get("kernel_source_sha256", {})
    if not isinstance(then, dict) or now.get("device_util.h") != then.get("device_util.h"):
        return None
    keep = {k: v for k, v in rec["kernels"].items()
            if now.get(v.get("source")) is not None
            and now.get(v.get("source")) == then.get(v.get("source"))}
    return dict(rec, kernels=keep) if keep else None


def kernel_bytes(rec, pattern):
    """Counter bytes per launch of the first kernel whose key matches the regex
    `pattern` in a traffic record (None if no kernel matches)."""
    if not rec:
        return None
    for k, v in rec["kernels"].items():
        if re.match(pattern, k):
            return v["bytes"]
    return None


def kernel_source(key: str) -> str:
    """Source file of a counted kernel of this library."""
    return "multi.hip" if key.startswith(("msell", "mbsell", "mtile", "mrow", "mvec", "minit",
                                          "mgrad")) else "solver.hip"
STEP_NAMES = {0: "plain SpMV y = A x (matrix from HBM)",
              1: "A step, iteration 1", 2: "A step (q = A p, p and x updates)",
              3: "G^T step, start-up", 4: "G^T step (t = G^T r, r update)",
              5: "G step, start-up", 6: "G step (z = G t + eps r)",
              7: "preconditioner tail (z = G t + eps r, no solver state)",
              8: "A product (separate form: q = A p, p.q)",
              9: "G^T product (separate form: t = G^T r)"}
MSTEP_NAMES = {0: "Y = M X (products of several vectors)", 1: "A step, iteration 1",
               2: "A step", 3: "G^T step", 4: "G step, start-up", 5: "G step",
               6: "A product (separate form)", 7: "G^T product (separate form)"}


def _pair_blocks(keys):
    """Column-block products run as csr_blk_step (the same kernel for every
    step) followed by blk_reduce<T, MODE>: name each csr_blk_step launch by
    the mode of the reduction that follows it, csr_blk_step<T, MODE>."""
    out = list(keys)
    for i, k in enumerate(out):
        if not k.startswith("csr_blk_step"):
            continue
        nxt = next((n for n in out[i + 1:] if n.startswith("blk_reduce<")), None)
        m = re.match(r"blk_reduce<(\w+), (\d+)>", nxt or "")
        if m:
            out[i] = f"csr_blk_step<{m.group(1)}, {m.group(2)}>"
    return out


def _counter_rows(run_dir):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"),
                                 recursive=True)):
        for r in csv.DictReader(open(path)):
            rows.append((int(r.get("Dispatch_Id", 0) or 0), _kernel_key(r["Kernel_Name"]),
                         float(r["Counter_Value"]), int(r.get("Grid_Size", 0))))
    rows.sort(key=lambda t: t[0])
    keys = _pair_blocks([k for _, k, _, _ in rows])
    out = {}
    for key, (_, _, v, g) in zip(keys, rows):
        out.setdefault(key, []).append((v, g))
    return out


def _kernel_key(nm):
    nm = nm.replace("void ", "").replace("sla::(anonymous namespace)::", "").replace("sla::", "")
    m = re.match(r"([\w:]+)(<[^>]*>)?", nm)
    return (m.group(1) + (m.group(2) or "")) if m else nm[:48]


def _describe(key):
    m = re.match(r"(sell_step|sell_win_step|csr_step|bsell_step|bsr3_step)<\w+, (\d+)", key)
    if m:
        return STEP_NAMES.get(int(m.group(2)), m.group(2))
    m = re.match(r"csr_blk_step<\w+, (\d+)>", key)
    if m:
        return "column blocks of the " + STEP_NAMES.get(int(m.group(1)), m.group(1))
    m = re.match(r"blk_reduce<\w+, (\d+)>", key)
    if m:
        return ("sum of the 8 column-block results, epilogue of the "
                + STEP_NAMES.get(int(m.group(1)), m.group(1)))
    m = re.match(r"(msell_step|mbsell_step|mtile_step|mrow_step)<\w+, (\d+), (\d+)", key)
    if m:
        return f"{MSTEP_NAMES.get(int(m.group(2)), m.group(2))}, K = {m.group(3)}"
    return {"vec_p_update": "p and x update pass", "vec_r_update": "r update pass, ||r||^2",
            "csr_grad": "dL/dA on the CSR pattern", "bsr3_grad": "dL/dA on the BSR pattern",
            "finalize_x": "last x update", "mvec_p": "P and X update pass (K columns)",
            "mvec_r": "R update pass (K columns)", "mgrad": "summed dL/dA (K columns)",
            "minit": "start-up (K columns)"}.get(key.split("<")[0], "")


def summarize_counters(fetch_dir, write_dir, l2_dir=None, workload="poisson3d_128",
                       run_args="--counters-workload", out_dir=None):
    """Turn the rocprofv3 --pmc runs of --counters-workload (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch; optionally TCC_HIT_sum and TCC_MISS_sum) into
    the per-kernel traffic summary profiles/traffic_<workload>.md and the record
    profiles/traffic_<workload>.json that the benchmark reads; the 256 MiB copy
    calibrates both byte counters."""
    fetch, write = _counter_rows(fetch_dir), _counter_rows(write_dir)
    l2 = _counter_rows(l2_dir) if l2_dir else {}
    copy_kib = 256 * 1024.0

    def calib(rows):
        vals = [v for k, lst in rows.items() if "copyBuffer" in k for v, g in lst]
        big = [v for v in vals if v > 0.25 * copy_kib]
        return copy_kib / statistics.median(big)
    fs, ws = calib(fetch), calib(write)
    kernels = {}
    for k in fetch:
        if k not in write or "copyBuffer" in k or "elementwise" in k.lower() or k.startswith("at::"):
            continue
        fk = statistics.fmean(v for v, _ in fetch[k])
        wk = statistics.fmean(v for v, _ in write[k])
        rec = {"dispatches": len(fetch[k]), "fetch_kib_raw": fk, "write_kib_raw": wk,
               "fetch_bytes": fk * 1024 * fs, "write_bytes": wk * 1024 * ws,
               "source": kernel_source(k)}
        rec["bytes"] = rec["fetch_bytes"] + rec["write_bytes"]
        kernels[k] = rec
    # L2 (TCC) hit rate: the HIT and MISS runs record one row per counter and dispatch
    if l2:
        import csv
        import glob
        rows = []
        for path in glob.glob(os.path.join(l2_dir, "**", "*counter_collection.csv"),
                              recursive=True):
            for r in csv.DictReader(open(path)):
                rows.append((int(r.get("Dispatch_Id", 0) or 0), _kernel_key(r["Kernel_Name"]),
                             r.get("Counter_Name", ""), float(r["Counter_Value"])))
        # one key per dispatch (two counter rows each), column-block passes
        # named by their reduction as for the byte counters
        ids = sorted({d for d, _, _, _ in rows})
        first = {}
        for d, k, _, _ in rows:
            first.setdefault(d, k)
        named = dict(zip(ids, _pair_blocks([first[d] for d in ids])))
        hm = {}
        for d_id, _, name, v in rows:
            d = hm.setdefault(named[d_id], {"hit": 0.0, "miss": 0.0})
            if "HIT" in name:
                d["hit"] += v
            elif "MISS" in name:
                d["miss"] += v
        for k, d in hm.items():
            if k in kernels and d["hit"] + d["miss"] > 0:
                kernels[k]["l2_hit_rate"] = d["hit"] / (d["hit"] + d["miss"])
    src_sha = kernel_source_shas()
    lines = ["| kernel | role | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) "
             "| written MB | total MB | L2 hit |", "|---|---|---|---|---|---|---|---|---|"]
    for k, r in sorted(kernels.items(), key=lambda kv: -kv[1]["bytes"] * kv[1]["dispatches"]):
        if r["bytes"] < 1e5:
            continue
        hit = f"{100 * r['l2_hit_rate']:.1f}%" if "l2_hit_rate" in r else "-"
        lines.append(f"| `{k}` | {_describe(k)} | {r['dispatches']} | {r['fetch_kib_raw']:,.1f} | "
                     f"{r['write_kib_raw']:,.1f} | {r['fetch_bytes'] / 1e6:.1f} | "
                     f"{r['write_bytes'] / 1e6:.1f} | {r['bytes'] / 1e6:.1f} | {hit} |")
    cmd = ("timeout -s KILL 300 rocprofv3 --pmc {c} --output-format csv -d {d} -o pmc -- "
           f"python -u bench.py {run_args}")
    cmds = ["    " + cmd.format(c="FETCH_SIZE", d=fetch_dir),
            "    " + cmd.format(c="WRITE_SIZE", d=write_dir)]
    if l2_dir:
        cmds.append("    " + cmd.format(c="TCC_HIT_sum TCC_MISS_sum", d=l2_dir))
    md = [f"# HBM traffic per launch of the PCG kernels, {workload}", "",
          "Counters from rocprofv3 --pmc runs of the benchmark's counter workload: a 256 MiB",
          "copy for calibration, then 20 forward and 20 adjoint PCG iterations (with dL/dA),",
          "20 lock-step iterations of each several-right-hand-side count, and 8 plain SpMVs",
          "alternating between two copies of A so that each streams its matrix from HBM.",
          "FETCH_SIZE and WRITE_SIZE are KiB per dispatch (averaged over the dispatches of",
          "each kernel); the copy of known size (256 MiB read, 256 MiB written) calibrates",
          f"fetched bytes by {fs:.3f} and written bytes by {ws:.3f}.  FETCH_SIZE counts what",
          "L2 fetches from the memory side, so Infinity Cache hits are included: an upper",
          "bound on HBM reads.  L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS) where taken.", "",
          "Commands (from the repository root, `export TMPDIR=/tmp`):", "", *cmds,
          f"    python bench.py --counter-summary {fetch_dir} {write_dir}"
          + (f" --l2-dir {l2_dir}" if l2_dir else "")
          + f" --workload-name {workload} --counters-args='{run_args}'", "", *lines, "",
          "Kernel sources (sha256): " + ", ".join(f"{f} {h}" for f, h in src_sha.items()) + ".",
          ""]
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    with open(os.path.join(out_dir, f"traffic_{workload}.md"), "w") as f:
        f.write("\n".join(md))
    with open(os.path.join(out_dir, f"traffic_{workload}.json"), "w") as f:
        json.dump({"workload": workload, "kernel_source_sha256": src_sha, "fetch_scale": fs,
                   "write_scale": ws, "kernels": kernels}, f, indent=1)
    print("\n".join(lines))


def _short_kernel(nm):
    import re
    nm = nm.replace("void ", "").replace("sla::(anonymous namespace)::", "").replace("sla::", "")
    m = re.match(r"([\w:]+)(<[^>]*>)?", nm)
    nm = (m.group(1) + (m.group(2) or "")) if m else nm
    return nm if len(nm) <= 48 else nm[:45] + "..."


def summarize_trace(trace_dir, bench_json=None, trace_args="--steps 2 --warmup 1 --no-cpu-baseline"):
    """Per-kernel table of a rocprofv3 --kernel-trace --stats run of this benchmark
    (profiles/kernel_trace_<workload>.md).  A launch counts as working when it
    runs longer than half its kernel's median launch: the others (1-5 us) are
    the early-out launches of a batch that ends after convergence."""
    import csv
    import glob
    recs = []
    for path in sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"),
                                 recursive=True)):
        for r in csv.DictReader(open(path)):
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            recs.append((t0, t1, _short_kernel(r["Kernel_Name"])))
    recs.sort()
    recs = [(t0, t1, k) for (t0, t1, _), k in zip(recs, _pair_blocks([k for _, _, k in recs]))]
    total = sum(t1 - t0 for t0, t1, _ in recs)
    by = {}
    for t0, t1, k in recs:
        by.setdefault(k, []).append((t1 - t0) / 1e3)
    rows = sorted(by.items(), key=lambda kv: -sum(kv[1]))
    cut = {k: 0.5 * statistics.median(d) for k, d in by.items()}
    lines = ["| kernel | calls | avg us (all) | % time | working launches | avg us (working) |",
             "|---|---|---|---|---|---|"]
    for k, d in rows[:16]:
        w = [v for v in d if v > cut[k]] or d
        lines.append(f"| `{k}` | {len(d)} | {statistics.fmean(d):.2f} | "
                     f"{100 * sum(d) * 1e3 / total:.2f} | {len(w)} | {statistics.fmean(w):.2f} |")
    step = [(t0, t1) for t0, t1, k in recs
            if k.split("<")[0] in ("sell_step", "sell_win_step", "csr_step", "bsell_step",
                                   "bsr3_step", "csr_blk_step", "blk_reduce")
            and (t1 - t0) / 1e3 > cut[k]]
    gaps = sorted(max(0, b0 - a1) / 1e3 for (a0, a1), (b0, b1) in zip(step, step[1:]))
    a_key = next((k for k, _ in rows
                  if re.match(r"(sell_win_step|sell_step|bsell_step|csr_step|bsr3_step)<\w+, (2|8),",
                              k)), None)
    a_work = [v for v in by.get(a_key, []) if v > cut[a_key]]
    blk_key = next((k for k, _ in rows if re.match(r"csr_blk_step<\w+, 8>", k)), None)
    if blk_key:
        # the A product on column blocks: each working csr_blk_step<T, 8> launch
        # plus the reduction launched right after it
        red = blk_key.replace("csr_blk_step", "blk_reduce")
        a_key = f"{blk_key} + {red}"
        a_work = [(a1 - a0 + b1 - b0) / 1e3
                  for (a0, a1, ka), (b0, b1, kb) in zip(recs, recs[1:])
                  if ka == blk_key and kb == red and (a1 - a0) / 1e3 > cut[blk_key]]
    cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d {d} -o bench -- "
           "python -u bench.py {a}").format(d=trace_dir, a=trace_args)
    rec = json.loads(open(bench_json).read().strip().splitlines()[-1]) if bench_json else None
    workload = rec["config"]["workload"] if rec else "poisson3d_128 (3D Poisson 128^3 fp64)"
    name = workload.split(" ")[0] + ("_f32" if rec and rec.get("dtype") == "f32" else "")
    md = [f"# Kernel trace of bench.py, {workload}", "",
          "Command (from the repository root, `export TMPDIR=/tmp`):",
          "", "    " + cmd, f"    python bench.py --trace-summary {trace_dir}"
          + (f" {bench_json}" if bench_json else "")
          + (f" --trace-args='{trace_args}'" if trace_args != "--steps 2 --warmup 1 "
             "--no-cpu-baseline" else ""), "",
          "Step kernels `<T, MODE, ...>`: MODE 2 = A step, 4 = G^T step, 6 = G step",
          "(1, 3, 5: their first-iteration / start-up forms, 0 = plain SpMV, 8 and 9 the",
          "A and G^T products of the separate iteration form); for `sell_step` NT =",
          "non-temporal matrix stream, I16 = 16-bit column offsets, U = slots per load",
          "batch.  \"calls\" counts every launch, including the launches of a batch that",
          "return at once after convergence; \"working launches\" keeps those longer than",
          "half the kernel's median launch (the ones that did the product).", "", *lines, ""]
    if a_work:
        md.append(f"The A step (`{a_key}`) averages {statistics.fmean(a_work):.2f} us per "
                  "working launch here.")
    if rec and rec["roofline"].get("avg_launch_us"):
        md.append("bench.py's own HIP-event measurement of the same kernel over its timed steps "
                  f"gave {rec['roofline']['avg_launch_us']:.2f} us (`roofline.avg_launch_us` of a "
                  "bench run of the same tree).")
    if gaps:
        md += ["", f"Gaps between consecutive working step kernels: median "
               f"{statistics.median(gaps):.2f} us, mean {statistics.fmean(gaps):.2f} us, 90th "
               f"percentile {gaps[int(0.9 * len(gaps))]:.2f} us over {len(gaps)} boundaries."]
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_{name}.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(lines))


def summarize_markers(trace_dir, log_path=None, name="powerlaw_20k",
                      run="-m preconditioned_cg_solver_amd.studies trace"):
    """profiles/marker_trace_<name>.md from a rocprofv3 --marker-trace
    --kernel-trace run with SLA_TRACE=1: each roctx range of the library, its
    duration and the kernels inside it, and the run's [sla] stderr lines."""
    import csv
    import glob
    mk = [r for path in glob.glob(os.path.join(trace_dir, "**", "*marker_api_trace.csv"),
                                  recursive=True) for r in csv.DictReader(open(path))]
    kr = [r for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"),
                                  recursive=True) for r in csv.DictReader(open(path))]
    kt = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in kr)
    lines = [f"# roctx ranges of the library (SLA_TRACE=1), {name}", "",
             "Commands (from the repository root, `export TMPDIR=/tmp`):", "",
             f"    SLA_TRACE=1 rocprofv3 --marker-trace --kernel-trace --output-format csv -d "
             f"{trace_dir} -o tr -- python -u {run} > LOG 2>&1",
             f"    python bench.py --marker-summary {trace_dir} LOG", "",
             "| range | duration ms | kernels inside | kernel time ms |", "|---|---|---|---|"]
    for r in sorted(mk, key=lambda r: int(r["Start_Timestamp"])):
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        ins = [(a, b) for a, b in kt if a >= t0 and b <= t1]
        lines.append(f"| `{r['Function']}` | {(t1 - t0) / 1e6:.3f} | {len(ins)} | "
                     f"{sum(b - a for a, b in ins) / 1e6:.3f} |")
    if log_path:
        lines += ["", "stderr lines of the same run:", ""]
        lines += ["    " + l.rstrip() for l in open(log_path) if l.startswith("[sla]")]
    with open(os.path.join(ROOT, "profiles", f"marker_trace_{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(p, w, min_seconds, expected_iters):
    """The oracle on the host cores doing the benchmark's step minus the handle
    set-up: the full forward PCG solve and the full adjoint solve on the same
    input, repeated until at least min_seconds have passed (at most 20 times).
    When one such pair would take more than three times min_seconds (the large
    workloads), both solves are cut at the same iteration cap instead, sized from
    a 3-iteration probe so that the pair takes about min_seconds: the rate is
    then iterations per second over truncated solves, said so in the sample.
    Then the same oracle on ONE thread pinned to one core of the affinity mask:
    a forward solve cut at the iteration count that takes about min_seconds / 2
    (the oracle's results are bitwise the same for any thread count)."""
    import oracle
    threads = oracle.num_threads()
    log(f"cpu oracle: forward + adjoint solves for >= {min_seconds:.0f} s, {threads} threads")
    # per-iteration cost from two short probes (3 and 6 iterations), so the
    # fixed cost of a solve (the oracle's own G^T build) is not counted per
    # iteration
    probe = []
    for m in (3, 6):
        t0 = time.perf_counter()
        oracle.pcg(p.A, p.G, p.eps, p.b, p.rtol, min(m, p.maxit))
        probe.append(time.perf_counter() - t0)
    per_it = max((probe[1] - probe[0]) / 3, 1e-9)
    fixed = max(probe[0] - 3 * per_it, 0.0)
    cap = p.maxit
    if 2 * fixed + per_it * expected_iters > 3 * min_seconds:
        cap = max(3, int((min_seconds / 2 - fixed) / per_it))
    its, reps = 0, 0
    t0 = time.perf_counter()
    while reps < 20 and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        x, st, it, _ = oracle.pcg(p.A, p.G, p.eps, p.b, p.rtol, cap)
        gx = w if w is not None else 2.0 * x      # dL/dx of <w, x>, or of sum(x^2)
        _, _, st2, it2, _ = oracle.adjoint(p.A, p.G, p.eps, x, gx, p.rtol, cap)
        its += it + it2
        reps += 1
    dt = time.perf_counter() - t0
    what = ("full forward PCG solve + full adjoint solve with dL/dA" if cap == p.maxit else
            f"forward PCG solve + adjoint solve with dL/dA, each cut at {cap} iterations "
            f"(the full pair runs {expected_iters} iterations on the GPU)")
    out = {"value": its / dt, "unit": "iters/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{reps} x ({what}) on the same {p.name} input, {its} iterations in "
                     f"{dt:.1f} s (each solve includes the oracle's own G^T build)"}
    # serial leg: one OpenMP thread, this thread pinned to one core
    mask = os.sched_getaffinity(0)
    core = min(mask)
    try:
        os.sched_setaffinity(0, {core})
        oracle.set_num_threads(1)
        log(f"cpu oracle: serial forward solve, 1 thread pinned to core {core}")
        t0 = time.perf_counter()
        _, _, it, _ = oracle.pcg(p.A, p.G, p.eps, p.b, p.rtol, min(3, p.maxit))
        per_it1 = (time.perf_counter() - t0) / max(it, 1)
        cap1 = max(3, min(p.maxit, int(0.5 * min_seconds / per_it1)))
        t0 = time.perf_counter()
        _, _, it1, _ = oracle.pcg(p.A, p.G, p.eps, p.b, p.rtol, cap1)
        dt1 = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(threads)
        os.sched_setaffinity(0, mask)
    out["serial_1core"] = {
        "value": it1 / dt1, "unit": "iters/s", "cores": 1,
        "sample": f"forward PCG solve cut at {cap1} iterations ({it1} run) on the same "
                  f"{p.name} input in {dt1:.1f} s, one thread pinned to core {core} "
                  f"(including the oracle's own G^T build)"}
    out["affinity_cores"] = len(mask)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", type=int, default=2, choices=range(5),
                    help="workload: 0 2D Poisson 32^2, 1 heat 512^2, 2 3D Poisson 128^3 "
                         "(the metric's), 3 elasticity BSR3 64^3, 4 power-law 4M")
    ap.add_argument("--size", type=int, default=None,
                    help="size parameter of the workload generator (grid edge; rows for 4)")
    ap.add_argument("--dtype", default="f64", choices=("f64", "f32"))
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum host time of the CPU-oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--spmv-reps", type=int, default=50)
    ap.add_argument("--multi-rhs", type=lambda v: [int(c) for c in v.split(",") if c],
                    default=[4, 8], help="right-hand-side counts of the multi-RHS lines "
                                         "(empty string: none)")
    ap.add_argument("--counters-workload", action="store_true",
                    help="short run for rocprofv3 --pmc: a 256 MiB copy (calibration) and "
                         "20 forward + 20 adjoint PCG iterations on the same input, then 8 "
                         "SpMVs alternating between two copies of A")
    ap.add_argument("--counter-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary under profiles/ from two rocprofv3 "
                         "--pmc runs of --counters-workload (no GPU needed)")
    ap.add_argument("--l2-dir", default=None,
                    help="with --counter-summary: a third run with TCC_HIT_sum TCC_MISS_sum")
    ap.add_argument("--workload-name", default="poisson3d_128",
                    help="with --counter-summary: the workload the runs measured")
    ap.add_argument("--counters-args", default="--counters-workload",
                    help="with --counter-summary: bench.py arguments of the counted runs")
    ap.add_argument("--trace-args", default="--steps 2 --warmup 1 --no-cpu-baseline",
                    help="bench.py arguments of the traced run (for the summary's command)")
    ap.add_argument("--marker-summary", nargs="+", metavar="DIR",
                    help="write profiles/marker_trace_powerlaw_20k.md from a rocprofv3 "
                         "--marker-trace run of the trace study (DIR [LOG])")
    ap.add_argument("--trace-summary", nargs="+", metavar="DIR",
                    help="write profiles/kernel_trace_<workload>.md from a rocprofv3 "
                         "--kernel-trace --stats run (and optionally a saved bench JSON line)")
    args = ap.parse_args()
    if args.marker_summary:
        summarize_markers(*args.marker_summary[:2])
        return
    if args.trace_summary:
        summarize_trace(*args.trace_summary[:2], trace_args=args.trace_args)
        return
    if args.counter_summary:
        summarize_counters(*args.counter_summary, l2_dir=args.l2_dir,
                           workload=args.workload_name, run_args=args.counters_args)
        return
    if args.steps < 1 or args.warmup < 0:
        print("bench.py needs --steps >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this solver runs on a single MI355X "
              "(multi-GPU sharding is described in the design notes, not built); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from preconditioned_cg_solver_amd import binding as B
    from preconditioned_cg_solver_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating inputs")
    p = I.make_problem(args.config, size=args.size)
    if args.dtype == "f32":
        p = p.astype("f32")
    sv = 4 if args.dtype == "f32" else 8
    tdt = torch.float32 if args.dtype == "f32" else torch.float64
    n, nnz_a, nnz_g = p.A.n, p.A.nnz, p.G.nnz
    ab = algorithmic_bytes(p.A, p.G, sv)
    bs = p.A.block_dim

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def mk(rp, ci, v, transpose=False):
        if bs == 1:
            return B.sla_csr_create(rp, ci, v, build_transpose=transpose)
        return B.sla_bsr_create(rp, ci, v, block_dim=bs, build_transpose=transpose)

    a_rp, a_ci, a_v = t(p.A.row_ptr), t(p.A.col_idx), t(p.A.vals)
    g_rp, g_ci, g_v = t(p.G.row_ptr), t(p.G.col_idx), t(p.G.vals)
    b = t(p.b)
    # dL/dx of the configuration's loss: <w, x> gives w, sum(x^2) gives 2x
    w = t(p.w) if p.w is not None else None
    x = torch.empty_like(b)
    grad_b = torch.empty_like(b)
    grad_vals = torch.empty(nnz_a, dtype=tdt, device=dev)
    work = None

    def loss_grad(xv):
        return w if w is not None else 2.0 * xv

    if args.counters_workload:
        src = torch.ones(32 * 1024 * 1024, dtype=torch.float64, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)                       # 256 MiB read + 256 MiB written
        torch.cuda.synchronize()
        A = mk(a_rp, a_ci, a_v)
        G = mk(g_rp, g_ci, g_v, transpose=True)
        work = B.workspace(A)
        B.sla_pcg_solve(A, G, p.eps, b, x=x, rtol=p.rtol, maxit=20, work=work)
        B.sla_pcg_adjoint(A, G, p.eps, x, loss_grad(x), rtol=p.rtol, maxit=20, grad_b=grad_b,
                          grad_vals=grad_vals, work=work)
        for k in args.multi_rhs:
            Bt = torch.from_numpy(np.random.default_rng(100 + k).standard_normal((n, k))).to(
                dev, tdt)
            B.sla_pcg_solve_multi(A, G, p.eps, Bt, rtol=p.rtol, maxit=20,
                                  work=B.workspace_multi(A, k, dev))
            del Bt
        # plain SpMV streaming its matrix from HBM: two copies of A alternately
        A2 = mk(a_rp.clone(), a_ci.clone(), a_v.clone())
        y = torch.empty_like(b)
        for _ in range(4):
            B.sla_spmv(A, b, y)
            B.sla_spmv(A2, b, y)
        torch.cuda.synchronize()
        log("counters workload done")
        return

    def step():
        nonlocal work
        A = mk(a_rp, a_ci, a_v)
        G = mk(g_rp, g_ci, g_v, transpose=True)
        if work is None:
            work = B.workspace(A)
        _, fi = B.sla_pcg_solve(A, G, p.eps, b, x=x, rtol=p.rtol, maxit=p.maxit, work=work)
        _, _, ai = B.sla_pcg_adjoint(A, G, p.eps, x, loss_grad(x), rtol=p.rtol, maxit=p.maxit,
                                     grad_b=grad_b, grad_vals=grad_vals, work=work)
        A.destroy()
        G.destroy()
        return fi, ai

    log(f"warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        fi, ai = step()
        log(f"forward iterations {fi.iterations}, adjoint iterations {ai.iterations}")

    # the A step's duration, live over the timed steps: events bracket the A
    # step of every PROF_EVERY-th iteration (a prime stride, so samples rotate
    # through the positions within the host's batches); each bracketed launch
    # leaves a ~4.5 us gap on either side in the queue, so every launch
    # bracketed would slow the measured solve by ~8%, every 23rd by ~0.4%
    B.sla_reset_profile()
    B.sla_set_profiling_stride(PROF_EVERY)
    B.sla_set_profiling(["a_step"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    total_iters = 0
    for k in range(args.steps):
        fi, ai = step()
        total_iters += fi.iterations + ai.iterations
        log(f"step {k + 1}/{args.steps} done")
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    B.sla_set_profiling(False)
    B.sla_set_profiling_stride(1)
    a_launches, a_ms = B.sla_get_profile("a_step")
    a_avg_s = a_ms / max(a_launches, 1) / 1e3

    # Outside the timed region: the parts of a step on their own.
    A = mk(a_rp, a_ci, a_v)
    G = mk(g_rp, g_ci, g_v, transpose=True)
    # the separate form's products on A's locality ordering run on column
    # blocks unless SLA_COLBLK=0
    colblk = (B.sla_mat_reordered(A) and not fused_iteration(p.A)
              and os.environ.get("SLA_COLBLK", "1") != "0")
    setup = []
    for _ in range(3):
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        H = mk(g_rp, g_ci, g_v, transpose=True)
        H2 = mk(a_rp, a_ci, a_v)
        torch.cuda.synchronize()
        setup.append(time.perf_counter() - s0)
        H.destroy()
        H2.destroy()
    solve_t = []
    for _ in range(3):
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        _, fi = B.sla_pcg_solve(A, G, p.eps, b, x=x, rtol=p.rtol, maxit=p.maxit, work=work)
        solve_t.append(time.perf_counter() - s0)
    tts = statistics.median(solve_t)
    # SpMV of A: kernel durations from the library's own fence-free events on
    # the launch stream (as for the roofline kernel)
    y = torch.empty_like(b)
    B.sla_spmv(A, b, y)
    torch.cuda.synchronize()
    B.sla_reset_profile()
    B.sla_set_profiling(["spmv"])
    for _ in range(args.spmv_reps):
        B.sla_spmv(A, b, y)
    torch.cuda.synchronize()
    nw, ms_w = B.sla_get_profile("spmv")
    spmv_s = ms_w / max(nw, 1) / 1e3
    # cold: a 1 GiB read-only pass before each call evicts A from L2 and the
    # 256 MB Infinity Cache without leaving dirty lines behind
    flush = torch.ones(128 * 1024 * 1024, dtype=torch.float64, device=dev)
    cold = []
    for _ in range(10):
        torch.cuda.synchronize()
        B.sla_reset_profile()
        flush.sum()
        B.sla_spmv(A, b, y)          # queued right behind the flush
        torch.cuda.synchronize()
        nc, ms_c = B.sla_get_profile("spmv")
        cold.append(ms_c / max(nc, 1) / 1e3)
    del flush
    spmv_cold_s = statistics.median(cold)
    # steady streaming: two handles over separate copies of A (2 x 183 MB, more
    # than the 256 MB Infinity Cache holds) called alternately, so each call
    # streams its matrix from HBM while x and y stay where the previous call
    # left them, as inside an iterative method
    A2 = mk(a_rp.clone(), a_ci.clone(), a_v.clone())
    for _ in range(4):
        B.sla_spmv(A, b, y)
        B.sla_spmv(A2, b, y)
    torch.cuda.synchronize()
    B.sla_reset_profile()
    for _ in range(args.spmv_reps // 2):
        B.sla_spmv(A, b, y)
        B.sla_spmv(A2, b, y)
    torch.cuda.synchronize()
    ns, ms_s = B.sla_get_profile("spmv")
    spmv_stream_s = ms_s / max(ns, 1) / 1e3
    B.sla_set_profiling(False)
    A2.destroy()

    # dL/dA alone (launched on torch's current stream, so torch events bracket
    # it): 10 back-to-back calls on the last adjoint's lambda and x
    B.sla_pattern_grad(A, grad_b, x, out=grad_vals)
    torch.cuda.synchronize()
    ge0, ge1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ge0.record()
    for _ in range(10):
        B.sla_pattern_grad(A, grad_b, x, out=grad_vals)
    ge1.record()
    torch.cuda.synchronize()
    grad_s = ge0.elapsed_time(ge1) / 10 / 1e3
    if bs == 1:
        grad_bytes = (sv + 4) * nnz_a + 4 * (n + 1) + 2 * sv * n
    else:
        grad_bytes = (9 * sv + 4) * p.A.nnzb + 4 * (p.A.n_block_rows + 1) + 2 * sv * n

    # several right-hand sides on the same operators (the single solve's b as
    # column 0, seeded N(0,1) columns after it): forward solves only
    multi = {}
    if args.multi_rhs:
        A = mk(a_rp, a_ci, a_v)
        G = mk(g_rp, g_ci, g_v, transpose=True)
        for k in args.multi_rhs:
            Bm = np.random.default_rng(100 + k).standard_normal((n, k))
            Bm[:, 0] = p.b
            Bt = torch.from_numpy(Bm).to(dev, tdt)
            Xt = torch.empty_like(Bt)
            wm = B.workspace_multi(A, k, dev)
            B.sla_pcg_solve_multi(A, G, p.eps, Bt, X=Xt, rtol=p.rtol, maxit=p.maxit, work=wm)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            _, infos = B.sla_pcg_solve_multi(A, G, p.eps, Bt, X=Xt, rtol=p.rtol, maxit=p.maxit,
                                             work=wm)
            torch.cuda.synchronize()
            tm = time.perf_counter() - t0
            its = [i.iterations for i in infos]
            multi[str(k)] = {"column_iterations": sum(its), "lockstep_iterations": max(its),
                             "ms": tm * 1e3, "column_iters_per_s": sum(its) / tm,
                             "vs_single_forward": (sum(its) / tm) / (fi.iterations / tts)}
            del Bt, Xt, wm
        A.destroy()
        G.destroy()

    # the A step's kernel: the one-workgroup solver (n <= 1024) has none of its own;
    # in the separate iteration form it is the bare product q = A p (p.q partials)
    has_a = a_launches > 0
    fused = fused_iteration(p.A)
    a_bytes = ab["a_step"] if fused else ab["spmv_A"]
    achieved = a_bytes / a_avg_s / 1e9 if has_a else None
    headline = args.config == 2 and args.dtype == "f64" and n == 128 ** 3
    workload = p.name + ("_f32" if args.dtype == "f32" else "")
    tr = traffic_if_current(workload)
    a_mode, gt_mode = (2, 4) if fused else (8, 9)
    step_re = r"(sell_win_step|sell_step|csr_step|bsell_step|bsr3_step)<\w+, {}[,>]"

    def step_bytes(mode):
        """Counter bytes of one step: its kernel, or on column blocks the
        block pass plus the reduction."""
        one = kernel_bytes(tr, step_re.format(mode))
        if one is not None:
            return one
        bp = kernel_bytes(tr, rf"csr_blk_step<\w+, {mode}>")
        br = kernel_bytes(tr, rf"blk_reduce<\w+, {mode}>")
        return bp + br if bp is not None and br is not None else None
    traffic = step_bytes(a_mode) if has_a else None
    physical = None
    if tr:
        parts = [step_bytes(a_mode), step_bytes(gt_mode), step_bytes(6)]
        if not fused:
            parts += [kernel_bytes(tr, k) for k in (r"vec_p_update<\w+, 2>", r"vec_r_update<")]
        sp = kernel_bytes(tr, step_re.format(0))
        it_bytes = sum(parts) if all(v is not None for v in parts) else None
        physical = {
            "source": f"profiles/traffic_{workload}.md (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                      "calibrated; Infinity Cache hits count as fetched)",
            "a_step": {"bytes": traffic, "GBps": traffic / a_avg_s / 1e9,
                       "frac": traffic / a_avg_s / 1e9 / HBM_PEAK_GBS} if traffic and has_a
                      else None,
            "spmv_hbm_stream": {"bytes": sp, "GBps": sp / spmv_stream_s / 1e9,
                                "frac": sp / spmv_stream_s / 1e9 / HBM_PEAK_GBS} if sp else None,
            "iteration": {"bytes": it_bytes, "GBps": it_bytes * fi.iterations / tts / 1e9,
                          "frac": it_bytes * fi.iterations / tts / 1e9 / HBM_PEAK_GBS}
                         if it_bytes else None}
    moved = moved_bytes_a_step(p.A, n, sv) if fused else None
    if fused and bs == 1 and slice_offset_slots(p.A) is not None and \
            os.environ.get("SLA_WIN", "1") != "0":
        a_kernel = (f"sell_win_step<{'double' if sv == 8 else 'float'}, A step> (q = A p with "
                    "p = z + beta p_old formed on the fly, near slots from an LDS window, "
                    "x += alpha_prev p_old, p.q partials)")
    elif fused and bs == 1:
        a_kernel = (f"sell_step<{'double' if sv == 8 else 'float'}, A step> (q = A p with "
                    "p = z + beta p_old formed on the fly, x += alpha_prev p_old, p.q partials)")
    elif fused:
        a_kernel = "bsell_step<A step> (BSR sliced ELL, p = z + beta p_old formed on the fly)"
    elif bs == 3:
        a_kernel = ("bsell_step<A product> (BSR sliced ELL, q = A p and p.q; p, x and r "
                    "updates in separate streaming passes)")
    elif colblk:
        a_kernel = ("csr_blk_step + blk_reduce<A product> (column blocks on the locality "
                    "ordering: q = A p per block of columns, the 8 results added with p.q; p, x "
                    "and r updates in separate streaming passes)")
    else:
        a_kernel = ("csr_step<A product> (LDS tiles, q = A p and p.q; p, x and r updates in "
                    "separate streaming passes)")
    describe = {
        0: "2D Poisson 5-point, 32^2 interior, CSR, PCG + factorised SPAI eps=3e-3, rtol=1e-10, "
           "forward + adjoint of sum(x^2)",
        1: "heat I + dt L5, 512^2, CSR, PCG + factorised SPAI eps=3e-3, rtol=1e-8, forward + "
           "adjoint",
        2: f"3D Poisson 7-point, {round(n ** (1 / 3))}^3 interior, fp64 CSR, PCG + factorised "
           "SPAI eps=3e-3, rtol=1e-10, forward + adjoint",
        3: "elasticity-like 27-point block system, 64^3 nodes x 3 dof, 3x3 BSR, PCG + "
           "factorised SPAI eps=3e-3, rtol=1e-8, forward + adjoint",
        4: "power-law random SPD, 4M rows, CSR, PCG + factorised SPAI eps=3e-3, rtol=1e-8, "
           "forward + adjoint"}
    iter_gbs = ab["iteration"] * fi.iterations / tts / 1e9
    spmv_gbs = ab["spmv_A"] / spmv_s / 1e9
    spmv_cold_gbs = ab["spmv_A"] / spmv_cold_s / 1e9
    spmv_stream_gbs = ab["spmv_A"] / spmv_stream_s / 1e9
    result = {
        "metric": METRIC if headline else
                  f"PCG iters/sec + SpMV HBM GB/s (% of peak), {p.name} {args.dtype}, 1 GPU",
        "value": total_iters / elapsed,
        "unit": "iters/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": f"{p.name} ({describe[args.config]})",
                   "n": n, "nnz_A": nnz_a, "nnz_G": nnz_g,
                   "iterations_forward": fi.iterations, "iterations_adjoint": ai.iterations,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm",
                     "kernel": a_kernel,
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": a_bytes,
                     "moved_bytes_per_launch": moved,
                     "moved_GBps": moved / a_avg_s / 1e9 if moved else None,
                     "avg_launch_us": a_avg_s * 1e6, "launches": a_launches,
                     "sampled_every": PROF_EVERY} if has_a else
                    {"bound": "latency", "note": "the whole solve runs in one workgroup "
                     "(n <= 1024): no per-step kernel to time"},
        "iteration": {"bytes": ab["iteration"], "GBps": iter_gbs, "frac": iter_gbs / HBM_PEAK_GBS,
                      "us_per_iteration": tts / fi.iterations * 1e6,
                      "time_to_solution_ms": tts * 1e3},
        "spmv": {"bytes": ab["spmv_A"],
                 "hbm_stream": {"GBps": spmv_stream_gbs, "frac": spmv_stream_gbs / HBM_PEAK_GBS,
                                "us": spmv_stream_s * 1e6},
                 "cold": {"GBps": spmv_cold_gbs, "frac": spmv_cold_gbs / HBM_PEAK_GBS,
                          "us": spmv_cold_s * 1e6},
                 "warm": {"GBps": spmv_gbs, "frac": spmv_gbs / HBM_PEAK_GBS,
                          "us": spmv_s * 1e6},
                 "note": "algorithmic bytes over the kernel's duration (library "
                         "events); hbm_stream = two copies of A called alternately (more "
                         "than the 256 MB Infinity Cache holds when A exceeds 128 MB), x and "
                         "y warm; cold = median of 10 calls, each after a 1 GiB read-only "
                         "flush of every cache (x included); warm = back-to-back calls "
                         "(A held in the Infinity Cache when it fits)"},
        "gradient": {"bytes": grad_bytes, "us": grad_s * 1e6,
                     "GBps": grad_bytes / grad_s / 1e9,
                     "frac": grad_bytes / grad_s / 1e9 / HBM_PEAK_GBS,
                     "note": "dL/dA = -lambda_i x_j on A's pattern (sla_pattern_grad), mean "
                             "of 10 back-to-back calls; bytes: column indices and row "
                             "pointers read, the gradient written, lambda and x read once"},
        "physical": physical,
        "setup_ms": statistics.median(setup) * 1e3,
        "multi_rhs": {"note": "k right-hand sides solved together on the same A and G "
                              f"(forward solves, {args.dtype}); column-iterations per second and the "
                              "ratio to the single-right-hand-side forward rate",
                      **multi} if multi else None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(p, p.w, args.cpu_seconds,
                                              fi.iterations + ai.iterations)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
