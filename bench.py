"""Benchmark of the fused inverse-RoPE + VHA postmix on one MI355X.

A step is one pass of the whole path over the production workload of
PaddleFleet PR #1772 (PR body item 1: sq=16384 tokens of a 64K context with
context_parallel_size=4, nh=64, nope=448, pe=64, a 1 GiB bf16 attention
output): the forward (postmix_fwd) and the backward (postmix_bwd: dO and dW
from one pass over dY and O), each reading its inputs from HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line.  `value` is the step's achieved HBM bandwidth: the
algorithmic bytes of the two calls (activations in and out, W, the cos/sin
rows touched, positions, dW) over the measured step time.  Per-op times come
from HIP events recorded on the stream the kernels run on.  The separate
backward entry points (postmix_bwd_dx, postmix_bwd_dw) are timed after the
steps and reported per op.  The oracle's CPU time on a bounded sample of the
same workload is reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "postmix fwd/bwd µs + achieved HBM GB/s (% peak), sq=16384 nh=64 d=512 bf16"
PEAK_GBPS = 8000.0  # MI355X HBM3E
KERNEL_SOURCE = os.path.join(ROOT, "rope_head_mixing_amd", "csrc", "postmix_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
# kernels behind each op at nh=64, d=512 (tiled path)
KERNELS_NH64 = {
    "fwd": "mix_part_kernel<64, 256, 8, false, 1, false>",
    "bwd": "bwd_fused_kernel<64, 256, 16, false, false, true> + dw_reduce_kernel",
    "bwd_dx": "mix_part_kernel<64, 256, 8, true, 1, false>",
    "bwd_dw": "dw_chunk_kernel<64, 128, false> + dw_reduce_kernel",
}
# the same at nh=3, d=512 (head-count sweep workload: 21 tokens per 64-row tile)
KERNELS_NH3 = {
    "fwd": "mix_part_kernel<64, 256, 8, false, 1, true>",
    "bwd": "bwd_fused_kernel<64, 256, 16, true, false, true> + dw_reduce_kernel",
    "bwd_dx": "mix_part_kernel<64, 256, 8, true, 1, true>",
    "bwd_dw": "dw_chunk_kernel<64, 128, true> + dw_reduce_kernel",
}
# the same at nh=128, d=512 (head-count sweep workload)
KERNELS_NH128 = {
    "fwd": "mix_part_kernel<128, 256, 8, false, 4, false>",
    "bwd": "bwd_fused_kernel<128, 128, 16, false, true, true> + dw_reduce_kernel",
    "bwd_dx": "mix_part_kernel<128, 256, 8, true, 4, false>",
    "bwd_dw": "dw_chunk_kernel<128, 128, false> + dw_reduce_kernel",
}
# nh=96 and nh=72 (96-row tiles and chunks; 72 with padding rows)
KERNELS_NH96 = {
    "fwd": "mix_part_kernel<96, 256, 6, false, 3, false>",
    "bwd": "bwd_fused_kernel<96, 256, 12, false, false, true> + dw_reduce_kernel",
    "bwd_dx": "mix_part_kernel<96, 256, 6, true, 3, false>",
    "bwd_dw": "dw_chunk_kernel<128, 128, true> + dw_reduce_kernel",
}
KERNELS_NH72 = {
    "fwd": "mix_part_kernel<96, 256, 6, false, 3, true>",
    "bwd": "bwd_fused_kernel<96, 256, 12, true, false, true> + dw_reduce_kernel",
    "bwd_dx": "mix_part_kernel<96, 256, 6, true, 3, true>",
    "bwd_dw": "dw_chunk_kernel<128, 128, true> + dw_reduce_kernel",
}
KERNELS_BY_WORKLOAD = {"prod": KERNELS_NH64, "fwd_1k": KERNELS_NH64, "sweep_nh3": KERNELS_NH3,
                       "sweep_nh128": KERNELS_NH128, "sweep_nh96": KERNELS_NH96, "sweep_nh72": KERNELS_NH72}
STEP_OPS = ("fwd", "bwd")          # the timed step
EXTRA_OPS = ("bwd_dx", "bwd_dw")   # the separate backward entry points, timed after
# The pages' own figures for this workload (another GPU; context only).
PAGES_CONTEXT = {
    "hardware": "1x B30Z (sm10.3)",
    "fwd_us_unfused_to_fused": [643.7, 459.4],
    "bwd_us_final_route_unfused_to_fused": [2700.1, 3012.3],
    "bwd_us_head_major_route_unfused_to_fused": [2699.4, 1828.9],
}


def kernel_source_sha() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    if doc.get("kernel_source_sha") != kernel_source_sha():
        return None
    entry = doc.get("kernels", {}).get(kernel_key)
    if not entry:
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(case, O, W, dY, pos, target_s: float):
    """The oracle, untouched, on the first S tokens of the workload (S sized
    from a short calibration so the timed run is about target_s seconds).
    The step's algorithmic bytes scale with the tokens, so the sample's rate is
    the full workload's; per op: the oracle's time extrapolated to the full
    workload, its GB/s over the op's algorithmic bytes and its GFLOP/s."""
    import oracle
    threads = oracle.default_threads()
    calls = {
        "fwd": lambda S: oracle.fwd(O[:S], W, pos[:S], case.theta, case.nope, case.pe, nthreads=threads),
        "bwd_dx": lambda S: oracle.bwd_dx(dY[:S], W, pos[:S], case.theta, case.nope, case.pe, nthreads=threads),
        "bwd_dw": lambda S: oracle.bwd_dw(dY[:S], O[:S], pos[:S], case.theta, case.nope, case.pe,
                                          nthreads=threads),
    }

    def one_pass(S):
        secs = {}
        for op, fn in calls.items():
            t0 = time.perf_counter()
            fn(S)
            secs[op] = time.perf_counter() - t0
        return secs

    cal = min(case.sq, 256)
    t_cal = sum(one_pass(cal).values())
    S = int(min(case.sq, max(cal, round(target_s / max(t_cal, 1e-6) * cal / 64) * 64)))
    secs = one_pass(S)
    t = sum(secs.values())
    frac = S / case.sq
    # the step (fwd + the single-call backward) moves these bytes; the oracle
    # computes the same outputs with its three functions
    alg = sum(case.algorithmic_bytes(op) for op in STEP_OPS) * frac
    per_op = {}
    for op, s in secs.items():
        per_op[op] = {"us_full_workload": round(s / frac * 1e6, 1),
                      "GBps": round(case.algorithmic_bytes(op) * frac / s / 1e9, 3),
                      "GFLOPs": round(case.flops() * frac / s / 1e9, 2)}
    return {
        "value": round(alg / t / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"fwd, dx and dW on the first {S} of {case.sq} tokens "
                  f"({t:.2f} s; the full step extrapolates to {t / frac * 1e6:.0f} us)",
        "seconds": round(t, 3),
        "us_per_full_step_extrapolated": round(t / frac * 1e6, 1),
        "ops": per_op,
    }


def summarize_profiles(trace_dir, fetch_dir, write_dir, command_note, out_prefix, timed=20,
                       kernels=None, traffic_file=True, copy_bytes=1 << 30):
    """Turn rocprofv3 outputs (kernel-trace --stats, --pmc FETCH_SIZE, --pmc
    WRITE_SIZE runs of this script) into profiles/<out_prefix>.md and (for
    the production workload, traffic_file=True) the per-launch HBM traffic
    file read by the benchmark.  `kernels` maps each op to its kernels
    (default: the production shape's); `copy_bytes` is the size of the
    benchmark's plain device copy of O for the workload (1 GiB in production).

    The counters are calibrated on the plain device copy of O that the
    benchmark runs (its known traffic: copy_bytes read, copy_bytes written)."""
    import collections
    import csv
    import glob

    def one(pattern):
        hits = glob.glob(pattern, recursive=True)
        if not hits:
            raise SystemExit(f"no file matches {pattern}")
        return hits[0]

    stats = list(csv.DictReader(open(one(os.path.join(trace_dir, "**", "*kernel_stats.csv")))))

    def counters(d, name):
        agg = collections.defaultdict(list)
        for r in csv.DictReader(open(one(os.path.join(d, "**", "*counter_collection.csv")))):
            if r["Counter_Name"] == name:
                agg[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]) * 1024)
        return {k: sum(v) / len(v) for k, v in agg.items()}

    fetch, write = counters(fetch_dir, "FETCH_SIZE"), counters(write_dir, "WRITE_SIZE")
    gib = float(1 << 30)
    # the copy of O: the copy kernel launch whose written bytes are largest
    copy_key = max((k for k in write if "copy" in k[0].lower()), key=lambda k: write[k])
    f_scale, w_scale = copy_bytes / fetch[copy_key], copy_bytes / write[copy_key]

    def short(name):
        return name.split("(")[0].replace("void ", "").replace("pm::", "")

    # per-kernel durations in launch order.  The timed steps are the last
    # `timed` repetitions of the step's kernel sequence (fwd then bwd) in the
    # longest back-to-back run of it; other kernels average their last `timed`
    # launches (each extra op is timed in a loop of its own, but some kernels
    # serve several ops, so that figure is indicative only).
    seq = sorted((int(r["Start_Timestamp"]), short(r["Kernel_Name"]),
                  (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
                 for r in csv.DictReader(open(one(os.path.join(trace_dir, "**", "*kernel_trace.csv")))))
    names = [x[1] for x in seq]
    kernels = KERNELS_NH64 if kernels is None else kernels
    pat = [k.strip() for op in STEP_OPS for k in kernels[op].split("+")]
    occ = [i for i in range(len(seq) - len(pat) + 1) if names[i:i + len(pat)] == pat]
    runs, cur = [], []
    for i in occ:
        if cur and i != cur[-1] + len(pat):
            runs.append(cur)
            cur = []
        cur.append(i)
    if cur:
        runs.append(cur)
    step_run = max(runs, key=len) if runs else []
    step_durs = collections.defaultdict(list)
    for i in step_run[-timed:]:
        for j, n in enumerate(pat):
            step_durs[n].append(seq[i + j][2])
    launches = collections.defaultdict(list)
    for _, n, dur in seq:
        launches[n].append(dur)
    rows = []
    for r in stats:
        n = short(r["Name"])
        tail = step_durs.get(n) or launches.get(n, [])[-timed:]
        rows.append((n, int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                     sum(tail) / len(tail) if tail else float("nan"),
                     float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    traffic = {}
    for (name, grid), fb in fetch.items():
        wb = write.get((name, grid), 0.0)
        traffic[short(name)] = {"fetch_bytes": fb * f_scale, "write_bytes": wb * w_scale,
                                "hbm_bytes_per_launch": fb * f_scale + wb * w_scale}
    ops = {op: [k.strip() for k in names.split("+")] for op, names in kernels.items()}
    doc = {"kernel_source_sha": kernel_source_sha(), "fetch_scale": f_scale, "write_scale": w_scale,
           "kernels": {}}
    for op, names in ops.items():
        present = [n for n in names if n in traffic]
        if present:
            doc["kernels"][op] = {
                "kernels": present,
                "hbm_bytes_per_launch": sum(traffic[n]["hbm_bytes_per_launch"] for n in present)}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    if traffic_file:
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(doc, f, indent=1)
            f.write("\n")
    lines = [f"# {out_prefix}: rocprofv3 kernel trace and HBM counters", "",
             "Commands (from the repository root on one MI355X):", "", "```", command_note.strip(),
             "```", "", f"Kernel source sha256[:16]: `{doc['kernel_source_sha']}`", "",
             "## Kernel durations (rocprofv3 --kernel-trace --stats)", "",
             f"`timed avg`: for the step's kernels ({' + '.join(pat)}), the mean over the "
             f"benchmark's {len(step_run[-timed:])} timed steps (the last {timed} repetitions of that "
             f"sequence in its back-to-back run of {len(step_run)}); for other kernels the mean of "
             f"their last {timed} launches.  `avg` includes warm-up launches.", "",
             "| kernel | calls | avg us | timed avg us | min us | max us |", "|---|---|---|---|---|---|"]
    lines += [f"| `{n}` | {c} | {a:.1f} | {ta:.1f} | {mn:.1f} | {mx:.1f} |" for n, c, a, ta, mn, mx in rows]
    lines += ["", "## HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)", "",
              f"Calibration on the benchmark's plain device copy of O, {copy_bytes / gib:.4f} GiB "
              f"(`{short(copy_key[0])}`): FETCH_SIZE x {f_scale:.3f}, WRITE_SIZE x {w_scale:.3f} "
              f"gives that read and written.", "",
              "| kernel | fetched GiB | written GiB | total GiB |", "|---|---|---|---|"]
    for n, t in sorted(traffic.items()):
        lines.append(f"| `{n}` | {t['fetch_bytes'] / gib:.4f} | {t['write_bytes'] / gib:.4f} | "
                     f"{t['hbm_bytes_per_launch'] / gib:.4f} |")
    path = os.path.join(ROOT, "profiles", f"{out_prefix}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)
    if traffic_file:
        print(TRAFFIC_FILE)


SQ_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
               "SQ_INSTS_LDS", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE")


def summarize_counters(pmc_dir, command_note, out_prefix, kernels=None, n_cu=256, n_simd=4, n_xcd=8):
    """Per-launch averages of the SQ_COUNTERS (one rocprofv3 --pmc run of this
    script) for the workload's kernels, with the rates derived from them, into
    profiles/<out_prefix>.md.  rocprofv3 sums each counter over its hardware
    instances, so the kernel's active cycles are GRBM_GUI_ACTIVE / XCDs; then
    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles * CUs * SIMDs), and LDS
    active and LDS bank-conflict cycles are per CU cycle."""
    import collections
    import csv
    import glob
    kernels = KERNELS_NH64 if kernels is None else kernels
    names = {k.strip() for v in kernels.values() for k in v.split("+")}
    hits = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not hits:
        raise SystemExit(f"no counter file under {pmc_dir}")
    # per dispatch: counter -> value (summed over the instances rocprofv3 reports)
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    kname = {}
    for r in csv.DictReader(open(hits[0])):
        short = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("pm::", "")
        if short not in names:
            continue
        per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
        kname[r["Dispatch_Id"]] = short
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for did, cv in per.items():
        for c, v in cv.items():
            agg[kname[did]][c].append(v)
    lines = [f"# {out_prefix}: rocprofv3 SQ counters", "", "Command (from the repository root on one MI355X):",
             "", "```", command_note.strip(), "```", "",
             f"Kernel source sha256[:16]: `{kernel_source_sha()}`", "",
             "Per-launch averages over the run's launches of each kernel (counters summed over their "
             "hardware instances).  Kernel cycles = GRBM_GUI_ACTIVE / 8 XCDs.  MFMA busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 256 CUs x 4 SIMDs); LDS active and LDS bank "
             "conflict = SQ_LDS_IDX_ACTIVE and SQ_LDS_BANK_CONFLICT / (cycles x 256 CUs); "
             "SQ_INSTS_VALU_MFMA_MOPS_BF16 counts units of 512 FLOPs.  Short kernels (the reduce) "
             "include the profiler's per-dispatch overhead in their cycles.",
             "", "| kernel | launches | " + " | ".join(SQ_COUNTERS) + " | MFMA busy | LDS active | LDS bank conflict |",
             "|---" * (len(SQ_COUNTERS) + 5) + "|"]
    for n in sorted(agg):
        a = {c: sum(v) / len(v) for c, v in agg[n].items()}
        gui = (a.get("GRBM_GUI_ACTIVE", 0.0) / n_xcd) or float("nan")
        mfma = a.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * n_cu * n_simd)
        lds = a.get("SQ_LDS_IDX_ACTIVE", 0.0) / (gui * n_cu)
        conf = a.get("SQ_LDS_BANK_CONFLICT", 0.0) / (gui * n_cu)
        cells = " | ".join(f"{a.get(c, float('nan')):.4g}" for c in SQ_COUNTERS)
        lines.append(f"| `{n}` | {len(next(iter(agg[n].values())))} | {cells} | {100 * mfma:.1f}% | "
                     f"{100 * lds:.1f}% | {100 * conf:.1f}% |")
    path = os.path.join(ROOT, "profiles", f"{out_prefix}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        # bench.py --summarize-counters PMC_DIR NAME COMMAND_NOTE_FILE [WORKLOAD]
        pmc_dir, name, note_file = sys.argv[2:5]
        workload = sys.argv[5] if len(sys.argv) > 5 else "prod"
        summarize_counters(pmc_dir, open(note_file).read(), name, kernels=KERNELS_BY_WORKLOAD[workload])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-profiles":
        # bench.py --summarize-profiles TRACE_DIR FETCH_DIR WRITE_DIR NAME COMMAND_NOTE_FILE [WORKLOAD]
        trace_dir, fetch_dir, write_dir, name, note_file = sys.argv[2:7]
        workload = sys.argv[7] if len(sys.argv) > 7 else "prod"
        from rope_head_mixing_amd import synthetic
        c = synthetic.CASES[workload]
        summarize_profiles(trace_dir, fetch_dir, write_dir, open(note_file).read(), name,
                           kernels=KERNELS_BY_WORKLOAD[workload], traffic_file=workload == "prod",
                           copy_bytes=c.sq * c.nh * c.d * 2)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prod",
                    help="prod (default) or another key of synthetic.CASES")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-target-seconds", type=float, default=12.0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}); this build has "
              "no multi-GPU path: forward and input gradient shard by tokens with no exchange, "
              "and the weight gradient would need one [nh,nh] fp32 sum across ranks.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from rope_head_mixing_amd import postmix as pm
    from rope_head_mixing_amd import synthetic

    pm.lib()  # raises if the HIP library is not built: no fallback
    torch.cuda.set_device(0)
    case = synthetic.CASES[args.workload]
    t0 = time.perf_counter()
    O, W, dY, pos = case.O(), case.W(), case.dY(), case.positions()
    gen_s = time.perf_counter() - t0

    def dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)

    dO_in, dW_in, ddY = dev_bf16(O), dev_bf16(W), dev_bf16(dY)
    dpos = torch.from_numpy(pos).cuda()
    cos, sin = pm.postmix_rope_table(case.theta, case.pe, int(pos.max()) + 1)
    Y = torch.empty_like(dO_in)
    dO = torch.empty_like(ddY)
    dW = torch.empty((case.nh, case.nh), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(256, pm.postmix_bwd_dw_workspace_bytes(case.sq, case.nh, case.nope, case.pe)),
                     dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    calls = {
        "fwd": lambda: pm.postmix_fwd(dO_in, dW_in, cos, sin, dpos, case.nope, case.pe, out=Y),
        "bwd": lambda: pm.postmix_bwd(ddY, dO_in, dW_in, cos, sin, dpos, case.nope, case.pe,
                                      out_dO=dO, out_dW=dW, workspace=ws),
        "bwd_dx": lambda: pm.postmix_bwd_dx(ddY, dW_in, cos, sin, dpos, case.nope, case.pe, out=dO),
        "bwd_dw": lambda: pm.postmix_bwd_dw(ddY, dO_in, cos, sin, dpos, case.nope, case.pe, out=dW,
                                            workspace=ws),
    }

    dist = [{}]  # op -> (median ms, min ms) of the timed passes

    def timed_loop(ops):
        """Warm up, then time args.steps passes of `ops`; events between calls."""
        for _ in range(args.warmup):
            for op in ops:
                calls[op]()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)]
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            ev[k][0].record()
            for i, op in enumerate(ops):
                calls[op]()
                ev[k][i + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        samples = {op: [ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(args.steps)]
                   for i, op in enumerate(ops)}
        ms = {op: float(np.mean(v)) for op, v in samples.items()}
        dist[0].update({op: (float(np.median(v)), float(np.min(v))) for op, v in samples.items()})
        return wall, ms

    # the unfused route (materialised inv_rope(O); rebuilt in the backward) and
    # the KV index remap at the pages' table shape [1 * 16384, 2176]
    calls["unfused_fwd"] = lambda: pm.unfused_fwd(dO_in, dW_in, cos, sin, dpos, case.nope, case.pe)
    calls["unfused_bwd"] = lambda: pm.unfused_bwd(ddY, dO_in, dW_in, cos, sin, dpos, case.nope, case.pe,
                                                  workspace=ws)
    kv_rows, kv_topk, kv_seqlen = 16384, 2176, 16384
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    kv_idx = torch.randint(-1, kv_seqlen, (kv_rows, kv_topk), generator=gen, device="cuda",
                           dtype=torch.int32)
    kv_out = torch.empty_like(kv_idx)
    calls["kv_remap"] = lambda: pm.postmix_kv_index_remap(kv_idx, kv_rows, kv_seqlen, out=kv_out)

    wall, per_op_ms = timed_loop(STEP_OPS)
    _, extra_ms = timed_loop(EXTRA_OPS)
    _, cmp_ms = timed_loop(("unfused_fwd", "unfused_bwd", "kv_remap"))
    per_op_ms.update(extra_ms)
    ops = list(STEP_OPS) + list(EXTRA_OPS)
    ms_per_step = wall * 1e3 / args.steps
    alg = {op: case.algorithmic_bytes(op) for op in ops}
    step_bytes = sum(alg[op] for op in STEP_OPS)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    op_report = {}
    for op in ops:
        gbps = alg[op] / (per_op_ms[op] * 1e-3) / 1e9
        med, mn = dist[0][op]
        op_report[op] = {"us": round(per_op_ms[op] * 1e3, 1), "GBps": round(gbps, 1),
                         "pct_peak": round(100 * gbps / PEAK_GBPS, 1),
                         "us_median": round(med * 1e3, 1), "us_min": round(mn * 1e3, 1),
                         "algorithmic_bytes": alg[op], "in_step": op in STEP_OPS}

    # device-to-device copy of the same 1 GiB, for an achievable-bandwidth reference
    src = dO_in.view(torch.int16)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 2 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
    del dst

    dominant = max(STEP_OPS, key=lambda op: per_op_ms[op])
    kernel_key = KERNELS_BY_WORKLOAD.get(args.workload, {}).get(dominant, dominant)
    achieved = alg[dominant] / (per_op_ms[dominant] * 1e-3) / 1e9
    roofline = {
        "bound": "hbm",
        "kernel": kernel_key,
        "achieved": round(achieved, 1),
        "peak": PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_GBPS, 4),
        "traffic": measured_traffic(dominant) if args.workload == "prod" else None,
    }

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{case.name}: postmix_fwd + postmix_bwd (dO and dW), O/dY [{case.sq}, {case.nh}, "
                        f"{case.nope}+{case.pe}] bf16 N(0,1), W [{case.nh},{case.nh}] = I + N(0,0.02), "
                        f"rotate-half RoPE theta={case.theta:g}, positions "
                        f"{int(pos[0])}..{int(pos[-1])}",
            "sq": case.sq, "nh": case.nh, "nope": case.nope, "pe": case.pe,
        },
        "ops": op_report,
        "pct_peak": round(100 * value / PEAK_GBPS, 1),
        "roofline": roofline,
        "unfused_route": {
            "fwd_us": round(cmp_ms["unfused_fwd"] * 1e3, 1),
            "bwd_us": round(cmp_ms["unfused_bwd"] * 1e3, 1),
            "fused_fwd_saves_pct": round(100 * (1 - per_op_ms["fwd"] / cmp_ms["unfused_fwd"]), 1),
            "fused_bwd_saves_pct": round(100 * (1 - per_op_ms["bwd"] / cmp_ms["unfused_bwd"]), 1),
            "extra_live_bytes": case.sq * case.nh * case.d * 2,
            "note": "same library's kernels: inv_rope(O) materialised in bf16, then the plain mix; "
                    "backward rebuilds it, plain dx and dW, then rope(dX)",
        },
        "kv_remap": {
            "table": [kv_rows, kv_topk],
            "us": round(cmp_ms["kv_remap"] * 1e3, 1),
            "GBps": round(2 * kv_rows * kv_topk * 4 / (cmp_ms["kv_remap"] * 1e-3) / 1e9, 1),
            "pct_peak": round(100 * 2 * kv_rows * kv_topk * 4 / (cmp_ms["kv_remap"] * 1e-3) / 1e9
                              / PEAK_GBPS, 1),
        },
        "copy_GBps": round(copy_gbps, 1),
        "input_generation_s": round(gen_s, 1),
        "context_pages": PAGES_CONTEXT,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case, O, W, dY, pos, args.cpu_target_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
