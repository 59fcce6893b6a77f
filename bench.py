"""Benchmark: tree-verify MLA-absorb attention step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload max_budget]

One step = the whole hot path over one batch: visibility masks from parent
pointers (derived inside the split kernel; --separate-visibility runs the
visibility kernel first instead), split-prefix verify attention + log-sum-exp
merge, and the accepted-path gather.  Inputs are seeded synthetic tensors of the
workload's shape, resident in HBM before timing starts.  Step i reads input copy
i mod n, in a ring that warm-up and timed steps continue without a break, and
n is chosen so that between two uses of one copy the other copies move more
than 320 MB: no step, timed or not, can find its inputs in the 256 MB Infinity
Cache, whatever --steps is.

Printed: one JSON line (metric, tree-tokens/s, ms per step, ...) with
  roofline     the verify-split kernel against the roofline that binds the
               workload (matrix cores when its flops per algorithmic byte are
               above the ridge point, 2.5 PFLOP/s / 8 TB/s, else HBM):
               algorithmic flops (or bytes) per launch / its mean launch time,
               timed with HIP events on the stream it runs on;
  cpu_baseline the float64 CPU oracle timed on the same workload (rank 0, N=1).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "verify-attn tree-tokens/sec + MFMA util % and HBM GB/s at q_len=65, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
INFINITY_CACHE_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="max_budget",
                    help="max_budget | batched | long_ctx | ragged_deep | tiny_fp32 (optionally :q1)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--kernel-only", action="store_true",
                    help="only run the verify-split kernel in the loop (for counter collection)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="run a plain device copy of MB megabytes --steps times (counter calibration)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--layout", type=int, default=0, help="force a workgroup layout (0: the planner's choice)")
    ap.add_argument("--split-keys", type=int, default=0, help="force a key split size (0: the planner's choice)")
    ap.add_argument("--separate-visibility", action="store_true",
                    help="build the masks with kdt_build_visibility in the step (default: the split kernel derives "
                         "them from the parents)")
    ap.add_argument("--partials-f32", action="store_true",
                    help="keep the split partials in float32 (default: the input dtype)")
    ap.add_argument("--merge-mode", type=int, default=0,
                    help="0: separate merge kernel (the library's default), "
                         "1: merge inside the split kernel when the launch allows")
    ap.add_argument("--schedule", type=int, default=0,
                    help="0: the library's choice, 1: splits, 2: the balanced schedule")
    ap.add_argument("--gang-size", type=int, default=0,
                    help="balanced schedule: row tiles per gang (0: the library's choice)")
    ap.add_argument("--no-length-hint", action="store_true",
                    help="do not tell the planner the sum of the prefix lengths (it then sizes the launch as if "
                         "every sequence had the longest length)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step directly instead of replaying HIP graphs (for counter runs)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_DB", "WRITE_DB", "CAL_FETCH_DB", "CAL_WRITE_DB"),
                    help="no GPU: turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE databases of a --kernel-only "
                         "--eager run and of a --copy-calibration run into "
                         "profiles/traffic_verify_split_<workload>.json")
    ap.add_argument("--trace-summary", nargs=2, metavar=("KERNEL_STATS_CSV", "BENCH_LOG"),
                    help="no GPU: print a markdown summary of a rocprofv3 --kernel-trace --stats --output-format "
                         "csv run of this script (its kernel_stats.csv and the bench line it printed)")
    ap.add_argument("--counter-summary", nargs="+", metavar="PMC_DB",
                    help="no GPU: print the split kernel's shader counters (means per dispatch) from rocprofv3 "
                         "--pmc databases of --kernel-only --eager runs, with derived rates")
    ap.add_argument("--calibration-mb", type=int, default=256,
                    help="size of the --copy-calibration run that --write-traffic reads")
    return ap.parse_args()


def pmc_kib_per_dispatch(db: str, counter: str, kernel_substr: str) -> float:
    """Mean of a rocprofv3 --pmc counter (summed over instances) per dispatch
    of the kernels whose name contains kernel_substr."""
    import sqlite3
    con = sqlite3.connect(db)
    names = {r[0]: r[1] for r in con.execute("select dispatch_id, name from kernels")}
    per = {}
    for cn, did, v in con.execute("select counter_name, dispatch_id, counter_value from pmc_events"):
        if cn == counter and kernel_substr in names.get(did, ""):
            per[did] = per.get(did, 0.0) + float(v)
    if not per:
        raise SystemExit(f"{db}: no {counter} values for kernels matching {kernel_substr!r}")
    return sum(per.values()) / len(per)


def write_traffic(args):
    """HBM bytes per launch of the split kernel from counter databases.
    FETCH_SIZE and WRITE_SIZE are in KiB; each is scaled by the ratio between
    the bytes a plain device copy of known size moves and what the same
    counter reports for it."""
    fetch_db, write_db, cal_fetch_db, cal_write_db = args.write_traffic
    n = args.calibration_mb << 20
    kernel = "verify_split_kernel"
    copy_kernel = "copyBuffer"
    cal_f = n / (pmc_kib_per_dispatch(cal_fetch_db, "FETCH_SIZE", copy_kernel) * 1024.0)
    cal_w = n / (pmc_kib_per_dispatch(cal_write_db, "WRITE_SIZE", copy_kernel) * 1024.0)
    fetch = pmc_kib_per_dispatch(fetch_db, "FETCH_SIZE", kernel) * 1024.0 * cal_f
    write = pmc_kib_per_dispatch(write_db, "WRITE_SIZE", kernel) * 1024.0 * cal_w
    rec = {"workload": args.workload, "kernel": kernel, "source_hash": source_hash(),
           "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "bytes_per_launch": fetch + write,
           "fetch_calibration": cal_f, "write_calibration": cal_w, "calibration_copy_bytes": n,
           "commands": [
               f"rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --workload {args.workload} --kernel-only --eager --no-cpu --steps 5 --warmup 1",
               f"rocprofv3 --pmc WRITE_SIZE -- python3 bench.py --workload {args.workload} --kernel-only --eager --no-cpu --steps 5 --warmup 1",
               f"rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --copy-calibration {args.calibration_mb} --steps 5",
               f"rocprofv3 --pmc WRITE_SIZE -- python3 bench.py --copy-calibration {args.calibration_mb} --steps 5",
               f"python3 bench.py --workload {args.workload} --write-traffic FETCH.db WRITE.db CAL_FETCH.db CAL_WRITE.db"]}
    out = os.path.join(ROOT, "profiles", f"traffic_verify_split_{args.workload.replace(':', '_')}.json")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def short_kernel_name(name: str) -> str:
    """Readable form of a (possibly mangled) kernel name: template
    arguments of the split and merge kernels spelled out."""
    m = re.match(r"_ZN3kdt19verify_split_kernelI(DF16b|f)Li(\d+)ELi(\d+)ELb([01])ELi(\d)ELb([01])E", name)
    if m:
        t, R, P, direct, cs, bal = m.groups()
        t = "bf16" if t == "DF16b" else "f32"
        return (f"verify_split_kernel<{t}, R={R}, P={P}, {'direct' if direct == '1' else 'partials'}, "
                f"layout {cs}{', balanced' if bal == '1' else ''}>")
    m = re.match(r"_ZN3kdt12merge_kernelI(DF16b|f)(DF16b|f)Lb([01])ELb([01])E", name)
    if m:
        o, pt, wide, gate = m.groups()
        dt = lambda x: "bf16" if x == "DF16b" else "f32"
        return (f"merge_kernel<out {dt(o)}, partials {dt(pt)}{', wide' if wide == '1' else ''}"
                f"{', gated' if gate == '1' else ''}>")
    m = re.match(r"_ZN3kdt18absorb_gemm_kernelILi(\d+)ELi(\d+)E", name)
    if m:
        return f"absorb_gemm_kernel<{m.group(1)}, {m.group(2)}>"
    return name.split("(")[0].replace("void ", "")


def trace_summary(args):
    import csv
    stats_csv, log = args.trace_summary
    rows = list(csv.DictReader(open(stats_csv)))
    bench = None
    for line in open(log):
        if line.startswith('{"metric"'):
            bench = json.loads(line)
    print("| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        print(f"| `{short_kernel_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    if bench:
        c, rf = bench["config"], bench["roofline"]
        print()
        print(f"Bench line of the same run: step {bench['ms_per_step'] * 1e3:.1f} us, "
              f"{bench['value']:.4g} {bench['unit']}; one kdt_verify_attn call {bench['verify_attn_us']['median']:.1f} us "
              f"(median); split kernel {rf['kernel_ms'] * 1e3:.1f} us by HIP events "
              f"({rf['bound']} bound: {rf['achieved']:.1f} of {rf['peak']:.0f} {rf['unit']}, "
              f"frac {rf['frac']:.3f}); layout {c['layout']}, {c['splits']} splits of {c['split_keys']} keys, "
              f"schedule {c.get('schedule', 'splits')}, partials {c['partials']}, merge {c['merge']}.")


def pmc_means(db: str, kernel_substr: str) -> dict:
    """Every counter of a rocprofv3 --pmc database: mean over the dispatches
    of the matching kernels of the counter summed over its instances."""
    import sqlite3
    con = sqlite3.connect(db)
    names = {r[0]: r[1] for r in con.execute("select dispatch_id, name from kernels")}
    per = {}
    for cn, did, v in con.execute("select counter_name, dispatch_id, counter_value from pmc_events"):
        if kernel_substr in names.get(did, ""):
            per.setdefault(cn, {}).setdefault(did, 0.0)
            per[cn][did] += float(v)
    return {cn: sum(d.values()) / len(d) for cn, d in per.items()}


def counter_summary(args):
    c = {}
    for db in args.counter_summary:
        c.update(pmc_means(db, "verify_split_kernel"))
    waves = c.get("SQ_WAVES", 0.0)
    print("| counter | mean per dispatch | per wave |")
    print("|---|---|---|")
    for k in sorted(c):
        print(f"| {k} | {c[k]:.4g} | {c[k] / waves:.4g} |" if waves else f"| {k} | {c[k]:.4g} | |")
    print()
    if "GRBM_GUI_ACTIVE" in c:
        cyc = c["GRBM_GUI_ACTIVE"] / 8.0
        print(f"* kernel cycles (GRBM_GUI_ACTIVE per XCD): {cyc:.0f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            print(f"* MFMA pipe busy over the whole kernel: SQ_VALU_MFMA_BUSY_CYCLES / (kernel cycles x 1024 SIMDs)"
                  f" = {c['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 1024):.3f}")
    if waves and "SQ_INSTS_MFMA" in c:
        print(f"* MFMA instructions per wave: {c['SQ_INSTS_MFMA'] / waves:.1f}")
    if waves and "SQ_INSTS_VALU" in c:
        print(f"* instructions per wave: {c['SQ_INSTS_VALU'] / waves:.0f} VALU (MFMA included), "
              f"{c.get('SQ_INSTS_SALU', 0) / waves:.0f} SALU, {c.get('SQ_INSTS_LDS', 0) / waves:.0f} LDS")
    if "SQ_WAVE_CYCLES" in c:
        wc = c["SQ_WAVE_CYCLES"]
        parts = []
        for k, what in (("SQ_ACTIVE_INST_ANY", "issuing"), ("SQ_WAIT_ANY", "waiting on any dependency"),
                        ("SQ_WAIT_INST_LDS", "waiting to issue an LDS instruction")):
            if k in c:
                parts.append(f"{what} {c[k] / wc:.3f}")
        print("* share of wave cycles: " + "; ".join(parts))
    if "SQ_LDS_BANK_CONFLICT" in c:
        print(f"* LDS bank conflicts: {c['SQ_LDS_BANK_CONFLICT']:.0f}")


def source_hash() -> str:
    """Hash of the sources the split-attention kernel is compiled from: stored
    traffic counts are used only while this still matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tree_verify_mla_kdt_amd", "csrc")
    for f in ("kdt_common.hpp", "kdt_verify.hip"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def visible_pairs(parents: np.ndarray, prefix_lens: np.ndarray, H: int) -> int:
    """Number of visible (query row, key) pairs: prefix keys plus ancestors-or-self."""
    B, q = parents.shape
    total = 0
    for b in range(B):
        depth = np.zeros(q, dtype=np.int64)
        for i in range(1, q):
            depth[i] = depth[parents[b, i]] + 1
        total += H * (q * int(prefix_lens[b]) + int(np.sum(depth + 1)))
    return total


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args)
        return
    if args.trace_summary:
        trace_summary(args)
        return
    if args.counter_summary:
        counter_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from tree_verify_mla_kdt_amd import kdt, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": args.steps}))
        return

    name, _, variant = args.workload.partition(":")
    cfg = synth.CONFIGS[name]
    if variant == "q1":
        cfg = synth.config_variant(cfg, q_len=1)
    inp = synth.generate(cfg)
    B, q, H, R, P = cfg.B, cfg.q_len, cfg.H, cfg.R, cfg.P

    def t_of(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # --- resident inputs: a ring of copies; between two uses of one copy the
    # other n - 1 move more than the Infinity Cache holds
    per_copy = inp.cache.nbytes + inp.q_lat.nbytes + inp.q_pe.nbytes
    n_copies = max(2, min(128, 1 + -(-(INFINITY_CACHE_BYTES + (64 << 20)) // per_copy)))
    base = {"cache": t_of(inp.cache), "q_lat": t_of(inp.q_lat), "q_pe": t_of(inp.q_pe)}
    copies = [{k: v.clone() for k, v in base.items()} for _ in range(n_copies)]
    parents = torch.from_numpy(inp.parents).to(dev)
    prefix_lens = torch.from_numpy(inp.prefix_lens).to(dev)
    accepted = torch.from_numpy(inp.accepted).to(dev)
    n_acc = torch.from_numpy(inp.n_accepted).to(dev)
    max_prefix = int(inp.prefix_lens.max())
    # the host knows its sequences' lengths: their sum sizes the launch
    total_prefix = 0 if args.no_length_hint else int(inp.prefix_lens.astype(np.int64).sum())
    sched = dict(schedule=args.schedule, gang_size=args.gang_size)
    W = (q + 63) // 64
    vis = torch.empty((B, q, W), dtype=torch.int64, device=dev)
    # masks: from kdt_build_visibility in the step, or derived by the split
    # kernel from the parents
    vis_arg, par_arg = (vis, None) if args.separate_visibility else (None, parents)
    depth = torch.empty((B, q), dtype=torch.int32, device=dev)
    out = torch.empty((B, q, H, R), dtype=base["q_lat"].dtype, device=dev)
    lse = torch.empty((B, q, H), dtype=torch.float32, device=dev)
    new_pl = torch.empty_like(prefix_lens)

    c0 = copies[0]
    desc, _, _ = kdt._verify_prepare(c0["q_lat"], c0["q_pe"], c0["cache"][..., :R], c0["cache"][..., R:],
                                     prefix_lens, vis_arg, cfg.softmax_scale, max_prefix, out, lse, None,
                                     args.split_keys, args.layout, args.partials_f32, par_arg, args.merge_mode,
                                     total_prefix_len=total_prefix, **sched)
    plan = kdt.verify_plan(desc)
    ws_bytes = max(int(plan.workspace_bytes), int(plan.partials_bytes))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)   # (merge counters start at zero)

    def step(i):
        c = copies[i % n_copies]
        if args.separate_visibility:
            kdt.build_visibility(parents, vis=vis, depth=depth)
        kdt.verify_attn(c["q_lat"], c["q_pe"], c["cache"][..., :R], c["cache"][..., R:], prefix_lens, vis_arg,
                        cfg.softmax_scale, max_prefix_len=max_prefix, out=out, lse=lse, workspace=ws,
                        split_keys=args.split_keys, layout=args.layout, partials_f32=args.partials_f32,
                        parents=par_arg, merge_mode=args.merge_mode, total_prefix_len=total_prefix, **sched)
        kdt.gather_accepted(c["cache"], prefix_lens, accepted, n_acc, q, new_prefix_lens=new_pl)

    def split_only(i):
        c = copies[i % n_copies]
        kdt.verify_partials(c["q_lat"], c["q_pe"], c["cache"][..., :R], c["cache"][..., R:], prefix_lens, vis_arg,
                            cfg.softmax_scale, max_prefix_len=max_prefix, workspace=ws,
                            split_keys=args.split_keys, layout=args.layout, partials_f32=args.partials_f32,
                            parents=par_arg, total_prefix_len=total_prefix, **sched)

    # Launches are replayed from HIP graphs: one graph runs the step once per
    # input copy, so host launch overhead stays out of the measured step time.
    def capture(fn, idx):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in idx:
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in idx:
                fn(i)
        return g

    kdt.build_visibility(parents, vis=vis, depth=depth)
    fn = split_only if args.kernel_only else step
    if args.eager:
        # counter runs: plain launches, no graphs, no timing report
        for i in range(args.warmup + args.steps):
            fn(i)
        torch.cuda.synchronize()
        print(json.dumps({"eager_steps": args.steps, "warmup": args.warmup, "workload": args.workload,
                          "kernel_only": bool(args.kernel_only)}), flush=True)
        return
    # one pass over the ring, the warm-up steps 0 .. W-1 and the timed steps
    # W .. W+K-1 (step i reads copy i mod n): captured first (each capture
    # runs its steps once), then replayed in ring order
    g_all = capture(fn, range(n_copies))
    g_warm = capture(fn, range(args.warmup)) if args.warmup > 0 else None
    g_timed = capture(fn, range(args.warmup, args.warmup + args.steps))
    g_all.replay()
    if g_warm is not None:
        g_warm.replay()
    torch.cuda.synchronize()

    # --- timed region: exactly K steps
    t0 = time.perf_counter()
    g_timed.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    # --- the dominant kernel alone, HIP events on the stream the graph runs on
    g_split = g_all if args.kernel_only else capture(split_only, range(n_copies))
    reps = max(1, -(-max(args.steps, 50) // n_copies))
    g_split.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    e0.record(cur)
    for _ in range(reps):
        g_split.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    split_ms = e0.elapsed_time(e1) / (reps * n_copies)

    # --- the same split kernel writing float32 partials (the bf16 partials
    # are the default for bf16 inputs; this is what the extra rounding saves)
    split_f32_us = None
    if cfg.dtype == "bf16" and not args.partials_f32:
        d32, _, _ = kdt._verify_prepare(c0["q_lat"], c0["q_pe"], c0["cache"][..., :R], c0["cache"][..., R:],
                                        prefix_lens, vis_arg, cfg.softmax_scale, max_prefix, out, lse, None,
                                        args.split_keys, args.layout, True, par_arg, total_prefix_len=total_prefix,
                                        **sched)
        p32 = kdt.verify_plan(d32)
        ws32 = torch.zeros(max(int(p32.partials_bytes), int(p32.workspace_bytes)), dtype=torch.uint8, device=dev)

        def split_only32(i):
            c = copies[i % n_copies]
            kdt.verify_partials(c["q_lat"], c["q_pe"], c["cache"][..., :R], c["cache"][..., R:], prefix_lens,
                                vis_arg, cfg.softmax_scale, max_prefix_len=max_prefix, workspace=ws32,
                                split_keys=args.split_keys, layout=args.layout, partials_f32=True, parents=par_arg,
                                total_prefix_len=total_prefix, **sched)
        g32 = capture(split_only32, range(n_copies))
        g32.replay()
        e0.record(cur)
        for _ in range(reps):
            g32.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        split_f32_us = e0.elapsed_time(e1) * 1e3 / (reps * n_copies)
        del g32, ws32

    # --- one verify call (split + merge) on its own: per-call mean over one
    # replay of a graph of n_copies calls, median and p90 over replays
    verify_us = None
    if not args.kernel_only:
        def verify_only(i):
            c = copies[i % n_copies]
            kdt.verify_attn(c["q_lat"], c["q_pe"], c["cache"][..., :R], c["cache"][..., R:], prefix_lens, vis_arg,
                            cfg.softmax_scale, max_prefix_len=max_prefix, out=out, lse=lse, workspace=ws,
                            split_keys=args.split_keys, layout=args.layout, partials_f32=args.partials_f32,
                            parents=par_arg, merge_mode=args.merge_mode, total_prefix_len=total_prefix, **sched)
        if args.separate_visibility:
            kdt.build_visibility(parents, vis=vis, depth=depth)
        g_ver = capture(verify_only, range(n_copies))
        g_ver.replay()
        samples = []
        for _ in range(max(20, reps)):
            e0.record(cur)
            g_ver.replay()
            e1.record(cur)
            torch.cuda.synchronize()
            samples.append(e0.elapsed_time(e1) * 1e3 / n_copies)
        verify_us = {"median": float(np.median(samples)), "p90": float(np.percentile(samples, 90)),
                     "samples": len(samples), "calls_per_sample": n_copies}

    # --- the visibility kernel on its own (the step derives the masks inside
    # the split kernel unless --separate-visibility)
    g_vis = capture(lambda i: kdt.build_visibility(parents, vis=vis, depth=depth), range(20))
    g_vis.replay()
    e0.record(cur)
    for _ in range(10):
        g_vis.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    vis_us = e0.elapsed_time(e1) * 1e3 / 200

    # --- greedy tree accept on the same trees (timed on its own: the step
    # above takes the accepted paths as input)
    tok_np, pred_np = synth.accept_inputs(inp.parents, 0)
    tok_d, pred_d = torch.from_numpy(tok_np).to(dev), torch.from_numpy(pred_np).to(dev)
    acc_d = torch.empty((B, q), dtype=torch.int32, device=dev)
    nacc_d = torch.empty((B,), dtype=torch.int32, device=dev)
    bonus_d = torch.empty((B,), dtype=torch.int32, device=dev)
    g_acc = capture(lambda i: kdt.tree_accept(parents, tok_d, pred_d, accepted=acc_d, n_accepted=nacc_d,
                                              bonus=bonus_d), range(20))
    g_acc.replay()
    e0.record(cur)
    for _ in range(10):
        g_acc.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    accept_us = e0.elapsed_time(e1) * 1e3 / 200

    # --- best-first tree build for the same batch and budget, from a drafter
    # shape of 16 draft positions x 8 candidates (timed on its own)
    tb_tok, tb_lp, tb_root = synth.tree_topk_inputs(B, 16, 8, 0)
    tb_tok, tb_lp, tb_root = (torch.from_numpy(x).to(dev) for x in (tb_tok, tb_lp, tb_root))
    g_tb = capture(lambda i: kdt.build_tree(tb_tok, tb_lp, tb_root, q), range(20))
    g_tb.replay()
    e0.record(cur)
    for _ in range(10):
        g_tb.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    tree_build_us = e0.elapsed_time(e1) * 1e3 / 200

    # --- the steps around the verify for the same batch (dn = dv = 128, the
    # MLA head dims of the model family): absorb_q + RoPE, cache append,
    # absorb_o, each timed on its own
    ab = synth.absorb_inputs(B, q, H, 128, P, R, 128, 0)
    ab = {k: torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16) for k, v in ab.items()}
    ab_depth = depth.clone()
    ab_qlat = torch.empty((B, q, H, R), dtype=torch.bfloat16, device=dev)
    ab_qpe = torch.empty((B, q, H, P), dtype=torch.bfloat16, device=dev)
    ab_o = torch.empty((B, q, H, 128), dtype=torch.bfloat16, device=dev)
    ab_cache = copies[0]["cache"]

    def time_graph(fn):
        g = capture(lambda i: fn(), range(20))
        g.replay()
        e0.record(cur)
        for _ in range(10):
            g.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / 200

    around_us = {
        "absorb_q": time_graph(lambda: kdt.absorb_q(ab["q"], ab["w_kc_t"], prefix_lens, ab_depth, 128, 50000.0,
                                                    q_lat=ab_qlat, q_pe=ab_qpe)),
        "append_tree_kv": time_graph(lambda: kdt.append_tree_kv(ab_cache, ab["c_kv_new"], ab["k_rope_new"],
                                                                prefix_lens, ab_depth, 50000.0)),
        "absorb_o": time_graph(lambda: kdt.absorb_o(ab["o_lat"], ab["w_vc"], o=ab_o)),
    }

    pairs = visible_pairs(inp.parents, inp.prefix_lens, H)
    flops = pairs * 2 * (R + P + R)                       # score over R+P, value over R
    esz = 2 if cfg.dtype == "bf16" else 4
    kv_bytes = int(np.sum(inp.prefix_lens.astype(np.int64) + q)) * (R + P) * esz
    alg_bytes = (kv_bytes + B * q * H * (R + P) * esz + B * q * H * R * esz + B * q * H * 4
                 + B * q * W * 8 + B * q * 4)
    peak_flops = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
    # the roofline that binds the workload: matrix cores above the ridge
    # point (peak flops / peak bandwidth), HBM below it
    mfma_bound = flops / alg_bytes >= peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        bound, unit, peak = "mfma", "TFLOP/s", peak_flops
        achieved = flops / (split_ms * 1e-3) / 1e12
    else:
        bound, unit, peak = "hbm", "GB/s", PEAK_HBM_GBS
        achieved = alg_bytes / (split_ms * 1e-3) / 1e9

    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_verify_split_{args.workload.replace(':', '_')}.json")
    if os.path.exists(tfile):
        rec = json.load(open(tfile))
        if rec.get("source_hash") == source_hash():
            traffic = rec.get("bytes_per_launch")

    tokens = B * q
    result = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tree-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tensors and random trees of the workload's shape)",
        "config": {"workload": f"{cfg.name}: {cfg.note}", "batch": B, "heads": H, "kv_lora_rank": R,
                   "rope_dim": P, "q_len": q, "prefix_len_max": max_prefix,
                   "split_keys": plan.split_keys, "splits": plan.max_splits, "layout": plan.layout,
                   "adaptive_splits": bool(plan.tiles_max), "length_hint": total_prefix,
                   "schedule": (f"balanced: {plan.gangs} gangs of {plan.gang_size} row tiles" if plan.gang_size
                                else "splits"),
                   "partials": "bf16" if plan.part_dtype == kdt.KDT_BF16 else "f32",
                   "merge": "direct" if plan.direct else ("fused" if plan.fused_merge else "separate kernel"),
                   "step": ("build_visibility + verify (split + merge) + gather_accepted" if args.separate_visibility
                            else "verify (split kernel deriving the masks from the parents + merge) + gather_accepted"),
                   "input_copies": n_copies, "kernel_only": bool(args.kernel_only)},
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel": "verify_split_kernel", "kernel_ms": split_ms,
                     "flops_per_launch": flops, "bytes_per_launch": alg_bytes, "visible_pairs": pairs,
                     "mfma_frac": flops / (split_ms * 1e-3) / 1e12 / peak_flops,
                     "hbm_frac": alg_bytes / (split_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "split_kernel_us_f32_partials": split_f32_us,
        "verify_attn_us": verify_us,
        "verify_tree_tokens_per_s": (B * q / (verify_us["median"] * 1e-6)) if verify_us else None,
        "mfma_util": flops / (ms_per_step * 1e-3) / 1e12 / peak,
        "hbm_gbs": alg_bytes / (ms_per_step * 1e-3) / 1e9,
        "hbm_frac": alg_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "algorithmic_bytes_per_step": alg_bytes,
        "build_visibility_us": vis_us, "tree_accept_us": accept_us,
        "tree_build_us": tree_build_us,
        "around_verify_us": around_us,
    }

    if not args.no_cpu and not args.kernel_only:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline(inp, budget_s: float):
    """Time the float64 oracle (as it stands) on the same workload: masks,
    verify attention and gather, repeated until ~budget_s of CPU work."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:      # threadpoolctl missing: numpy's BLAS uses every core by default
        threads = os.cpu_count() or 1
    cfg = inp.cfg
    R = cfg.R
    cache = inp.f64("cache")
    ql, qp = inp.f64("q_lat"), inp.f64("q_pe")
    n = 0
    t0 = time.perf_counter()
    while True:
        vis, _ = oracle.build_visibility(inp.parents)
        oracle.verify_attn(ql, qp, cache[..., :R], cache[..., R:], inp.prefix_lens, vis, cfg.softmax_scale)
        oracle.gather_accepted(inp.cache, inp.prefix_lens, inp.accepted, inp.n_accepted)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / n
    return {"value": cfg.B * cfg.q_len / per, "unit": "tree-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"full {cfg.name} workload (masks + verify + gather), {n} repetitions, {el:.1f} s",
            "seconds_per_step": per}


if __name__ == "__main__":
    main()
