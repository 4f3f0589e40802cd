"""Benchmark: batch-invariant selected-token log-probabilities + mismatch stats.

One *step* is the whole hot path over one batch already resident in HBM:
``tim_logprob_forward`` (fused bf16 LM-head contraction, online log-sum-exp,
gather, chunk merge) followed by ``tim_mismatch_stats`` (delta, ratio,
k1/k2/k3, truncated IS, per-sequence rejection, batch aggregates) on the
Qwen3-8B-shaped workload: N=8192 tokens in 16 sequences of 512, D=4096,
V=151936, bf16 inputs, fp32 accumulation.

Prints ONE JSON line on stdout.  Diagnostics go to stderr.  Also reported:
the stats pass on 2^28 tokens (HBM bandwidth), the extra metrics (extreme
rate, relative difference, ratio quantiles, |delta| p95) on the workload and
on 2^28 tokens, the backward (dh, dW) on the workload, the PPO surrogate on
2^28 tokens, the price of batch invariance against the free schedule, and
the fp64 oracle timed on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_F32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
MFMA_SUMMARY = os.path.join(ROOT, "profiles", "lmhead_mfma_counters.json")
METRIC = "selected-token logprobs/s at D=4096,V=151936 (bf16) + MFMA util; batch-invariant"
PMC_SUMMARY = os.path.join(ROOT, "profiles", "lmhead_bf16_qwen3_8b_counters.json")
# the sources the head kernel is built from (its tiles, pipeline and chunking)
LMHEAD_SRC = tuple(os.path.join(ROOT, "invariant_logprobs_amd", "csrc", f)
                   for f in ("lmhead.hip", "mfma_pipe.h", "tim_internal.h"))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_digest(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(launch_unit):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if absent or taken on a different kernel source."""
    try:
        with open(PMC_SUMMARY) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    if s.get("kernel_source_sha256_16") != source_digest(LMHEAD_SRC):
        return None
    if s.get("launch_unit") != launch_unit:
        return None
    return s.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="oracle rows for the CPU baseline (0: ~15 s of work)")
    ap.add_argument("--stats-log2", type=int, default=28)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the stats-scale and invariance-cost measurements")
    ap.add_argument("--profile-pass", action="store_true",
                    help="short run for a rocprofv3 counter pass: a 1 GiB copy kernel "
                         "(calibrates the byte counters), then the timed steps only")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of --profile-pass runs into the traffic summary and exit")
    ap.add_argument("--stats-scale-only", action="store_true",
                    help="run only the stats pass at 2^stats-log2 tokens (for a kernel trace)")
    ap.add_argument("--extras-scale-only", action="store_true",
                    help="run only the extra metrics at 2^stats-log2 tokens (for a kernel trace)")
    ap.add_argument("--backward-only", action="store_true",
                    help="run only the backward on the workload (for a kernel trace)")
    ap.add_argument("--ex-only", action="store_true",
                    help="only the tempered / entropy / RMSNorm scoring measurements")
    ap.add_argument("--ppo-scale-only", action="store_true",
                    help="run only the surrogate at 2^stats-log2 tokens (for a kernel trace)")
    ap.add_argument("--mfma-from", nargs=2, metavar=("COUNTER_CSV", "KERNEL_TRACE_CSV"),
                    help="turn a rocprofv3 --pmc MfmaUtil ... pass of --profile-pass (counter "
                         "and kernel-trace CSV) into the matrix-unit summary and exit")
    ap.add_argument("--mfma-out", default=MFMA_SUMMARY)
    ap.add_argument("--traffic-out", default=PMC_SUMMARY)
    ap.add_argument("--small-batch-only", action="store_true",
                    help="only the forward at b = 1 .. 64 tokens (for a kernel trace)")
    ap.add_argument("--trace-summary", nargs=2, metavar=("KERNEL_TRACE_DIR", "OUT_MD"),
                    help="write a markdown summary of a rocprofv3 --kernel-trace --stats "
                         "output directory (this library's kernels per call, launch "
                         "shapes) and exit")
    ap.add_argument("--title", default="", help="--trace-summary: heading")
    ap.add_argument("--notes", default="", help="--trace-summary: workload text")
    ap.add_argument("--traffic-command", default="",
                    help="the commands that made the CSV files, recorded in the summary")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(args.traffic_from[0], args.traffic_from[1], args.traffic_out,
                      args.traffic_command)
        return
    if args.mfma_from:
        write_mfma(args.mfma_from[0], args.mfma_from[1], args.mfma_out, args.traffic_command)
        return
    if args.trace_summary:
        write_trace_summary(args.trace_summary[0], args.trace_summary[1], args.title,
                            args.notes, args.traffic_command)
        return
    if args.profile_pass:
        args.no_extras = True
        args.no_cpu_baseline = True
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(scoring shards by rows with no exchange; only the ~21 batch aggregates "
              "of the statistics would need one)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import invariant_logprobs_amd as tim
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    torch.cuda.set_device(0)
    if args.profile_pass:
        copy_calibration(torch)
    if args.stats_scale_only:
        print(json.dumps(stats_scale(tim, workloads, torch, np, args.stats_log2)), flush=True)
        return
    if args.extras_scale_only:
        tau = workloads.SPECS["qwen3_8b"].tok_tau
        print(json.dumps(extras_scale(tim, workloads, torch, np, args.stats_log2, tau)),
              flush=True)
        return
    if args.ppo_scale_only:
        print(json.dumps(ppo_scale(tim, torch, np, args.stats_log2)), flush=True)
        return
    name = "qwen3_8b"
    log(f"generating workload {name}")
    wl = workloads.make(name, device=dev)
    if args.small_batch_only:
        print(json.dumps(small_batch_measure(tim, wl, torch, np)), flush=True)
        return
    if args.backward_only:
        res = backward_measure(tim, wl, torch, np)
        del wl
        torch.cuda.empty_cache()
        res["fp32_head"] = backward_measure(tim, workloads.make("fp32_head", device=dev), torch,
                                            np, reps=3)
        print(json.dumps(res), flush=True)
        return
    if args.ex_only:
        print(json.dumps(scoring_ex_measure(tim, workloads, wl, torch, np)), flush=True)
        return
    sp = wl.spec
    n, d, v = sp.n, sp.d, sp.v
    torch.cuda.synchronize()

    # preallocated outputs and workspaces: the timed region only launches
    lt = torch.empty(n, dtype=torch.float32, device=dev)
    ws_lp = torch.empty(tim.logprob_workspace_bytes(n, d, v, tim.TIM_BF16), dtype=torch.uint8,
                        device=dev)
    ws_st = torch.empty(max(1, tim.stats_workspace_bytes(n, sp.n_seqs)), dtype=torch.uint8,
                        device=dev)

    def step():
        tim.tim_logprob_forward(wl.h, wl.w, wl.ids, out=lt, workspace=ws_lp)
        return tim.tim_mismatch_stats(lt, wl.logp_rollout, wl.mask, wl.cu_seqlens,
                                      tis_clip=sp.clip_c, seq_bounds=(sp.seq_lo, sp.seq_hi),
                                      workspace=ws_st)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        tim.tim_logprob_forward(wl.h, wl.w, wl.ids, out=lt, workspace=ws_lp)
        ev[i][1].record(stream)
        res = tim.tim_mismatch_stats(lt, wl.logp_rollout, wl.mask, wl.cu_seqlens,
                                     tis_clip=sp.clip_c, seq_bounds=(sp.seq_lo, sp.seq_hi),
                                     workspace=ws_st)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_lp = [ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]     # ms
    t_st = [ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]
    ms_step = wall * 1e3 / K
    value = n / (ms_step / 1e3)
    lp_avg = float(np.mean(t_lp))
    flops = 2.0 * n * d * v
    achieved = flops / (lp_avg / 1e3) / 1e12
    log(f"step {ms_step:.3f} ms (wall), forward avg {lp_avg:.3f} ms "
        f"(p10 {np.percentile(t_lp, 10):.3f}, p90 {np.percentile(t_lp, 90):.3f}), "
        f"stats avg {np.mean(t_st) * 1e3:.1f} us, {achieved:.1f} TFLOP/s")
    bsum = tim.batch_dict(res["batch"])
    log(f"is_approx_k3_kl {bsum['is_approx_k3_kl']:.3e}, reject_frac {bsum['reject_frac']}")
    if args.profile_pass:
        # the fp32 head's kernel in the same counter pass
        fp32_head_measure(tim, workloads, torch, np, reps=3, compare_bf16=False)

    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": sp.desc, "n_tokens": n, "hidden": d, "vocab": v,
                   "sequences": sp.n_seqs, "schedule": "invariant",
                   "accumulation": "fp32"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic(f"{name}:N={n}"),
                     "kernel": "lmhead8w_kernel (bf16) + lse_merge (one forward call)",
                     "flops_per_launch": flops, "avg_launch_ms": lp_avg,
                     **measured_mfma(LMHEAD_KERNEL)},
        "stats_step_us": float(np.mean(t_st)) * 1e3,
    }

    if not args.no_extras:
        out["fp32_head"] = fp32_head_measure(tim, workloads, torch, np)
        out["small_batch"] = small_batch_measure(tim, wl, torch, np)
        out["scoring_ex"] = scoring_ex_measure(tim, workloads, wl, torch, np)
        out["backward"] = backward_measure(tim, wl, torch, np)
        out["backward"]["fp32_head"] = backward_measure(
            tim, workloads.make("fp32_head", device=dev), torch, np, reps=3)
        out["ppo"] = ppo_scale(tim, torch, np, args.stats_log2)
        out["extras"] = extras_measure(tim, workloads, wl, torch, np, args.stats_log2)
        out["stats_scale"] = stats_scale(tim, workloads, torch, np, args.stats_log2)
        out["invariance_cost"] = invariance_cost(tim, wl, torch, np)
        out["dsv3"] = dsv3_measure(tim, workloads, torch, np)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, np, args.cpu_rows)

    print(json.dumps(out), flush=True)


def fp32_head_measure(tim, workloads, torch, np, reps=5, compare_bf16=True):
    """The fp32 LM head (fp32 h and W, fp32 MFMA; N = 4096 in 8 sequences of
    512, D = 4096, V = 151936) against the fp32 matrix peak, and the same
    rows rounded to bf16 through the bf16 kernel: the distribution of
    |logp_bf16 - logp_fp32| over all 4096 tokens."""
    wl = workloads.make("fp32_head", device="cuda")
    sp = wl.spec
    n, d, v = sp.n, sp.d, sp.v
    lt = torch.empty(n, dtype=torch.float32, device="cuda")
    ws = torch.empty(tim.logprob_workspace_bytes(n, d, v, tim.TIM_F32), dtype=torch.uint8,
                     device="cuda")
    fn = lambda: tim.tim_logprob_forward(wl.h, wl.w, wl.ids, out=lt, workspace=ws)
    ms = time_calls(fn, torch, np, reps=reps, warm=1)
    flops = 2.0 * n * d * v
    tf = flops / (ms / 1e3) / 1e12
    log(f"fp32 head: {ms:.3f} ms, {tf:.1f} TFLOP/s ({tf / PEAK_F32_MFMA_TFLOPS:.1%} of fp32 MFMA peak)")
    res = {"workload": sp.desc, "ms": ms, "flops": flops, "achieved_TFLOPs": tf,
           "peak_TFLOPs": PEAK_F32_MFMA_TFLOPS, "frac": tf / PEAK_F32_MFMA_TFLOPS,
           "tokens_per_s": n / (ms / 1e3), "kernel": "lmhead_partials_kernel (fp32) + lse_merge",
           **measured_mfma(LMHEAD_F32_KERNEL)}
    if compare_bf16:
        hb, wb = wl.h.to(torch.bfloat16), wl.w.to(torch.bfloat16)
        l16 = tim.tim_logprob_forward(hb, wb, wl.ids)
        dd = (l16.double() - lt.double()).abs().cpu().numpy()
        res["bf16_vs_fp32_abs_dlogp"] = {"tokens": n, "mean": float(dd.mean()),
                                         "p99": float(np.quantile(dd, 0.99)),
                                         "max": float(dd.max())}
        log(f"|logp_bf16 - logp_fp32|: mean {dd.mean():.3e} p99 {np.quantile(dd, 0.99):.3e} "
            f"max {dd.max():.3e}")
        del hb, wb, l16
    del wl, ws, lt
    torch.cuda.empty_cache()
    return res


SMALL_BATCHES = (1, 7, 16, 32, 64)


def small_batch_measure(tim, wl, torch, np):
    """The forward on the first b rows of the workload: at these sizes the
    call is bound by reading W once (V D 2 bytes), so it is reported as a
    fraction of HBM bandwidth."""
    sp = wl.spec
    res = {}
    wbytes = 2.0 * sp.v * sp.d
    for b in SMALL_BATCHES:
        h, ids = wl.h[:b], wl.ids[:b]
        out = torch.empty(b, dtype=torch.float32, device="cuda")
        ws = torch.empty(tim.logprob_workspace_bytes(b, sp.d, sp.v, tim.TIM_BF16),
                         dtype=torch.uint8, device="cuda")
        ms = time_calls(lambda: tim.tim_logprob_forward(h, wl.w, ids, out=out, workspace=ws),
                        torch, np, reps=20)
        gbs = wbytes / (ms / 1e3) / 1e9
        res[str(b)] = {"ms": ms, "w_bytes": wbytes, "achieved_GBs": gbs,
                       "frac_hbm": gbs / PEAK_HBM_GBS}
        log(f"small batch b={b}: {ms * 1e3:.1f} us, {gbs:.0f} GB/s of W ({gbs / PEAK_HBM_GBS:.1%} of HBM)")
    return res


def measured_mfma(kernel_key):
    """Matrix-unit counters of one kernel from the committed summary, or {}
    if absent or taken on a different kernel source."""
    try:
        with open(MFMA_SUMMARY) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return {}
    if s.get("kernel_source_sha256_16") != source_digest(LMHEAD_SRC):
        return {}
    k = s.get("kernels", {}).get(kernel_key)
    if not k:
        return {}
    return {"mfma_busy": k["mfma_util"], "clock_ghz": k.get("clock_ghz"),
            "mfma_counters": os.path.relpath(MFMA_SUMMARY, ROOT)}


def write_mfma(counter_csv, trace_csv, out_path, command):
    """Per-kernel matrix-unit utilisation (rocprofv3's MfmaUtil: MFMA-busy
    cycles summed over SIMDs / (GUI-active cycles x SIMDs)), the GUI-active
    cycles per XCC divided by the kernel's duration (the clock it ran at), and
    the MFMA work the counters saw against the algorithmic 2 N D V."""
    import csv

    import numpy as np
    vals = {}
    with open(counter_csv, newline="") as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            for key in (LMHEAD_KERNEL, LMHEAD_F32_KERNEL):
                if key in name:
                    d = vals.setdefault(key, {}).setdefault(row.get("Dispatch_Id", ""), {})
                    d[row["Counter_Name"]] = float(row["Counter_Value"])
    durs = {}
    with open(trace_csv, newline="") as f:
        for row in csv.DictReader(f):
            for key in (LMHEAD_KERNEL, LMHEAD_F32_KERNEL):
                if key in row["Kernel_Name"]:
                    durs.setdefault(key, []).append(
                        (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e9)
    summary = {"command": command, "kernel_source_sha256_16": source_digest(LMHEAD_SRC),
               "definition": "mfma_util = sum of SQ_VALU_MFMA_BUSY_CYCLES / (max GRBM_GUI_ACTIVE "
                             "x SIMD count) (rocprofv3 MfmaUtil); clock_ghz = GRBM_GUI_ACTIVE "
                             "summed over the 8 XCDs / 8 / kernel duration",
               "kernels": {}}
    algo = {LMHEAD_KERNEL: 2.0 * 8192 * 4096 * 151936, LMHEAD_F32_KERNEL: 2.0 * 4096 * 4096 * 151936}
    for key, dispatches in vals.items():
        util = [d["MfmaUtil"] for d in dispatches.values() if "MfmaUtil" in d]
        gui = [d["GRBM_GUI_ACTIVE"] for d in dispatches.values() if "GRBM_GUI_ACTIVE" in d]
        mops = [d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + d.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0)
                for d in dispatches.values()]
        dur = sorted(durs.get(key, []))
        k = {"dispatches": len(dispatches), "mfma_util": float(np.mean(util)) / 100.0 if util else None,
             "mfma_flops_per_dispatch": float(np.mean(mops)) * 512 if mops else None,
             "algorithmic_flops": algo[key]}
        if gui and dur:
            med = dur[len(dur) // 2]
            k["duration_ms_median"] = med * 1e3
            k["clock_ghz"] = float(np.mean(gui)) / 8 / med / 1e9
        summary["kernels"][key] = k
    with open(out_path, "w") as f:
        json.dump(summary, f, indent=1)
        f.write("\n")
    print(json.dumps(summary, indent=1))


def write_trace_summary(trace_dir, out_path, title, notes, command):
    """Markdown from a rocprofv3 --kernel-trace --stats directory: the stats
    table of this library's kernels (tim::), every call's duration in launch
    order, and each kernel's launch shape (grid, workgroup, LDS, registers,
    scratch)."""
    import csv
    import glob
    import re

    def one(pattern):
        hits = glob.glob(os.path.join(trace_dir, "**", pattern), recursive=True)
        if not hits:
            raise SystemExit(f"no {pattern} under {trace_dir}")
        return hits[0]

    def short(name):
        name = re.sub(r"\(anonymous namespace\)::", "", name)
        name = name.replace("void ", "", 1)
        return name.split("(")[0]

    trace = list(csv.DictReader(open(one("*kernel_trace.csv"), newline="")))
    lines = [f"# {title}", ""]
    if notes:
        lines += [notes, ""]
    lines += ["Command (repo root):", "", f"    {command}", "",
              "## Kernel durations (this library's kernels; all calls, warmup included)", "",
              "| kernel | calls | avg us | min us | max us | total ms |",
              "|---|---:|---:|---:|---:|---:|"]
    agg, other = {}, 0.0
    for r in trace:
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if "tim::" in r["Kernel_Name"]:
            agg.setdefault(short(r["Kernel_Name"]), []).append(dur)
        else:
            other += dur * 1e3
    for k, us in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k}` | {len(us)} | {sum(us) / len(us):.1f} | {min(us):.1f} | "
                     f"{max(us):.1f} | {sum(us) / 1e3:.3f} |")
    lines += ["", f"Other kernels (torch: input generation, reference ops): {other / 1e6:.3f} ms in total.",
              "", "## Per call (us, launch order) and launch shape", ""]
    per = {}
    for r in trace:
        if "tim::" not in r["Kernel_Name"]:
            continue
        k = short(r["Kernel_Name"])
        d = per.setdefault(k, {"us": [], "row": r})
        d["us"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    for k, d in per.items():
        us = d["us"]
        r = d["row"]
        med = sorted(us)[len(us) // 2]
        shown = ", ".join(f"{x:.0f}" if x >= 100 else f"{x:.1f}" for x in us[:40])
        more = f" ... ({len(us)} calls)" if len(us) > 40 else ""
        lines += [f"- `{k}`: median {med:.1f} us; {shown}{more}",
                  f"  grid {r['Grid_Size_X']} work-items, workgroup {r['Workgroup_Size_X']}, "
                  f"LDS {r['LDS_Block_Size']} B, VGPR {r['VGPR_Count']}, AGPR {r['Accum_VGPR_Count']}, "
                  f"SGPR {r['SGPR_Count']}, scratch {r['Scratch_Size']} B"]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


COPY_BYTES = 1 << 30          # bytes read and bytes written by the calibration kernel
COPY_KERNEL = "bitwise_not_kernel"   # one coalesced 4-byte read and write per element
LMHEAD_KERNEL = "lmhead8w_kernel<false, false>"
LMHEAD_F32_KERNEL = "lmhead_partials_kernel<false, 0>"
STATS_KERNEL = "stats_stream_kernel"
EXTRAS_KERNEL = "xsel_pass_kernel"


def copy_calibration(torch):
    """A plain elementwise kernel over 1 GiB in and 1 GiB out, three times:
    the counters' reading for it gives bytes-per-counted-byte."""
    n = COPY_BYTES // 4
    src = torch.zeros(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def _counter_values(path, counter):
    """Counter_Value (KiB) of every dispatch, in order, per kernel of interest."""
    import csv
    vals = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            for key in (COPY_KERNEL, LMHEAD_KERNEL, STATS_KERNEL, EXTRAS_KERNEL):
                if key in name:
                    # one row per dispatch (values already summed over the chip)
                    vals.setdefault(key, []).append(float(row["Counter_Value"]))
    return vals


def _counter_means(path, counter):
    """Mean Counter_Value (KiB) per dispatch for each kernel name of interest."""
    return {k: (sum(v) / len(v), len(v)) for k, v in _counter_values(path, counter).items()}


def write_traffic(fetch_csv, write_csv, out_path, command):
    """Per-dispatch bytes of the LM-head kernel (bench run) or of the stats
    kernel (stats-only run), each counter scaled by its reading for the copy
    kernel of known size."""
    fr = _counter_means(fetch_csv, "FETCH_SIZE")
    wr = _counter_means(write_csv, "WRITE_SIZE")
    if COPY_KERNEL not in fr or COPY_KERNEL not in wr:
        raise SystemExit("no copy-calibration dispatches in the counter files")
    rf = fr[COPY_KERNEL][0] * 1024 / COPY_BYTES      # counted bytes per true byte read
    wf = wr[COPY_KERNEL][0] * 1024 / COPY_BYTES
    summary = {
        "copy_calibration": {"kernel": "torch.bitwise_not over 2^28 int32 "
                                       "(1 GiB read, 1 GiB written)",
                             "fetch_factor": rf, "write_factor": wf,
                             "dispatches": fr[COPY_KERNEL][1]},
        "command": command,
    }
    for key, tag in ((LMHEAD_KERNEL, "lmhead"), (STATS_KERNEL, "stats_stream")):
        if key in fr and key in wr:
            summary[tag] = {"kernel": key, "fetch_kib_raw": fr[key][0],
                            "write_kib_raw": wr[key][0],
                            "fetch_bytes": fr[key][0] * 1024 / rf,
                            "write_bytes": wr[key][0] * 1024 / wf,
                            "dispatches": fr[key][1]}
    # the radix-select pass: passes after the last target is resolved return
    # at once, so the bytes of every dispatch are kept, in launch order
    fv = _counter_values(fetch_csv, "FETCH_SIZE").get(EXTRAS_KERNEL)
    wv = _counter_values(write_csv, "WRITE_SIZE").get(EXTRAS_KERNEL)
    if fv and wv:
        summary["extras_pass"] = {"kernel": EXTRAS_KERNEL,
                                  "fetch_bytes_per_dispatch": [x * 1024 / rf for x in fv],
                                  "write_bytes_per_dispatch": [x * 1024 / wf for x in wv],
                                  "dispatches": len(fv)}
    if "lmhead" in summary:
        summary["kernel"] = LMHEAD_KERNEL
        summary["kernel_source_sha256_16"] = source_digest(LMHEAD_SRC)
        summary["launch_unit"] = "qwen3_8b:N=8192"
        summary["hbm_bytes_per_launch"] = summary["lmhead"]["fetch_bytes"] + \
            summary["lmhead"]["write_bytes"]
    with open(out_path, "w") as f:
        json.dump(summary, f, indent=1)
        f.write("\n")
    print(json.dumps(summary, indent=1))


def time_calls(fn, torch, np, reps=10, warm=2):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(s)
        fn()
        b.record(s)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def stats_scale(tim, workloads, torch, np, log2n):
    n = 1 << log2n
    log(f"stats at 2^{log2n} tokens")
    lt, lr, mask, cu = workloads.stats_scale(n, seed=7, device="cuda")
    s = cu.numel() - 1
    ws = torch.empty(tim.stats_workspace_bytes(n, s), dtype=torch.uint8, device="cuda")
    fn = lambda: tim.tim_mismatch_stats(lt, lr, mask, cu, seq_bounds=(math.log(0.99),
                                        math.log(1.01)), workspace=ws)
    ms = time_calls(fn, torch, np)
    # algorithmic bytes: lt, lr (4 B) + mask (1 B) per token, cu_seqlens,
    # per-sequence outputs (3 int32, 5 fp64, 2 u8), the batch vector
    algo = 9 * n + 4 * (s + 1) + s * (12 + 40 + 2) + 8 * len(tim.BATCH_FIELDS)
    gbs = algo / (ms / 1e3) / 1e9
    log(f"stats 2^{log2n}: {ms:.3f} ms, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%} of HBM)")
    del lt, lr, mask, cu, ws
    torch.cuda.empty_cache()
    return {"tokens": n, "sequences": s, "ms": ms, "algorithmic_bytes": algo,
            "achieved_GBs": gbs, "peak_GBs": PEAK_HBM_GBS, "frac": gbs / PEAK_HBM_GBS,
            "tokens_per_s": n / (ms / 1e3)}


XQ_RATIO = (0.01, 0.5, 0.99)   # ratio quantiles of the mismatch metric table
XQ_ABS = (0.95,)                # p95 of |delta|


def extras_measure(tim, workloads, wl, torch, np, log2n):
    """tim_mismatch_extras (extreme rate, mean relative difference, ratio
    quantiles, |delta| p95) on the bench workload and on 2^log2n tokens."""
    sp = wl.spec
    ws = torch.empty(tim.extras_workspace_bytes(sp.n), dtype=torch.uint8, device="cuda")
    fn = lambda: tim.tim_mismatch_extras(wl.logp_sampler, wl.logp_rollout, wl.mask,
                                         tok_tau=sp.tok_tau, ratio_q=XQ_RATIO, abs_q=XQ_ABS,
                                         workspace=ws)
    us_small = time_calls(fn, torch, np, reps=20) * 1e3
    log(f"extras: {us_small:.1f} us at N={sp.n}")
    out = extras_scale(tim, workloads, torch, np, log2n, sp.tok_tau)
    out.update({"workload_us": us_small, "workload_tokens": sp.n})
    return out


def extras_scale(tim, workloads, torch, np, log2n, tok_tau):
    """The extra metrics on 2^log2n tokens of the statistics workload.
    Algorithmic bytes are the inputs read once (9 B per token); the radix
    select reads them once per pass, so its fraction of that bound shows the
    price of the passes."""
    n = 1 << log2n
    lt, lr, mask, _ = workloads.stats_scale(n, seed=7, device="cuda")
    wsl = torch.empty(tim.extras_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    fl = lambda: tim.tim_mismatch_extras(lt, lr, mask, tok_tau=tok_tau, ratio_q=XQ_RATIO,
                                         abs_q=XQ_ABS, workspace=wsl)
    ms = time_calls(fl, torch, np, reps=5)
    res = tim.extras_dict(fl(), len(XQ_RATIO), len(XQ_ABS))
    algo = 9 * n + 8 * len(tim.EXTRAS_FIELDS)
    gbs = algo / (ms / 1e3) / 1e9
    log(f"extras 2^{log2n}: {ms:.3f} ms, {gbs:.0f} GB/s of one input read "
        f"({gbs / PEAK_HBM_GBS:.1%}); ratio q {res['ratio_q']}, |d| p95 {res['abs_q'][0]:.4g}, "
        f"extreme {res['extreme_frac']:.3e}")
    del lt, lr, mask, wsl
    torch.cuda.empty_cache()
    return {"tokens": n, "ms": ms, "algorithmic_bytes": algo, "achieved_GBs": gbs,
            "peak_GBs": PEAK_HBM_GBS, "frac": gbs / PEAK_HBM_GBS, "ratio_q": list(XQ_RATIO),
            "abs_q": list(XQ_ABS), "tok_tau": tok_tau}


def dsv3_measure(tim, workloads, torch, np):
    """The largest configuration, a DeepSeek-V3-shaped head (N = 32768 in 64
    log-normal sequences, D = 7168, V = 129280, bf16): forward (logits,
    log-sum-exp, gather, merge) and the mismatch statistics, each timed
    alone, median of 5 calls."""
    wl = workloads.make("dsv3", device="cuda")
    sp = wl.spec
    n, d, v = sp.n, sp.d, sp.v
    lt = torch.empty(n, dtype=torch.float32, device="cuda")
    ws_lp = torch.empty(tim.logprob_workspace_bytes(n, d, v, tim.TIM_BF16), dtype=torch.uint8,
                        device="cuda")
    ws_st = torch.empty(max(1, tim.stats_workspace_bytes(n, sp.n_seqs)), dtype=torch.uint8,
                        device="cuda")
    fwd = lambda: tim.tim_logprob_forward(wl.h, wl.w, wl.ids, out=lt, workspace=ws_lp)
    ms = time_calls(fwd, torch, np, reps=5, warm=1)
    st = lambda: tim.tim_mismatch_stats(lt, wl.logp_rollout, wl.mask, wl.cu_seqlens,
                                        tis_clip=sp.clip_c, seq_bounds=(sp.seq_lo, sp.seq_hi),
                                        workspace=ws_st)
    ms_st = time_calls(st, torch, np, reps=5, warm=1)
    flops = 2.0 * n * d * v
    tf = flops / (ms / 1e3) / 1e12
    log(f"dsv3 forward: {ms:.3f} ms, {tf:.1f} TFLOP/s ({tf / PEAK_BF16_TFLOPS:.1%} of bf16 peak); "
        f"stats {ms_st * 1e3:.1f} us")
    del wl, ws_lp, ws_st, lt
    torch.cuda.empty_cache()
    return {"workload": sp.desc, "forward_ms": ms, "stats_us": ms_st * 1e3,
            "tokens_per_s": n / ((ms + ms_st) / 1e3), "flops": flops, "achieved_TFLOPs": tf,
            "peak_TFLOPs": PEAK_BF16_TFLOPS, "frac": tf / PEAK_BF16_TFLOPS}


def backward_measure(tim, wl, torch, np, reps=5):
    """tim_logprob_backward on the workload with a dense upstream gradient:
    the logits recomputed (2 N D V FLOP), dh = dz W and dW = dz^T h (2 N D V
    each), against the dense MFMA peak of the inputs' type (bf16, or fp32 for
    the FP32 head)."""
    sp = wl.spec
    n, d, v = sp.n, sp.d, sp.v
    f32 = wl.h.dtype == torch.float32
    dtype = tim.TIM_F32 if f32 else tim.TIM_BF16
    peak = PEAK_F32_MFMA_TFLOPS if f32 else PEAK_BF16_TFLOPS
    _, lse, _ = tim.tim_logprob_forward(wl.h, wl.w, wl.ids, return_lse=True)
    g = torch.Generator(device="cuda").manual_seed(11)
    grad = torch.randn(n, generator=g, device="cuda", dtype=torch.float32) / n
    ws = torch.empty(tim.backward_workspace_bytes(n, d, v, dtype), dtype=torch.uint8,
                     device="cuda")
    dh = torch.empty(n, d, dtype=torch.float32, device="cuda")
    dw = torch.empty(v, d, dtype=torch.float32, device="cuda")
    fn = lambda: tim.tim_logprob_backward(wl.h, wl.w, wl.ids, lse, grad, dw=dw, workspace=ws)
    ms = time_calls(fn, torch, np, reps=reps, warm=1)
    flops = 3 * 2.0 * n * d * v
    tf = flops / (ms / 1e3) / 1e12
    kind = "fp32" if f32 else "bf16"
    log(f"backward ({kind}): {ms:.3f} ms, {tf:.1f} TFLOP/s ({tf / peak:.1%} of {kind} peak), "
        f"workspace {ws.numel() / 2**30:.2f} GiB")
    res = {"ms": ms, "flops": flops, "achieved_TFLOPs": tf, "peak_TFLOPs": peak,
           "frac": tf / peak, "tokens": n, "hidden": d, "vocab": v, "dtype": kind,
           "workspace_GiB": ws.numel() / 2**30}
    del ws, dh, dw
    torch.cuda.empty_cache()
    return res


EX_TAU = 0.7
NORM_EPS = 1e-6


def scoring_ex_measure(tim, workloads, wl, torch, np, norm_log2_rows=18):
    """tim_logprob_forward_ex on the workload at temperature 0.7 with the
    entropy, without and with the RMSNorm in front (2 N D V FLOP each, like
    the plain forward), and tim_rmsnorm alone on the workload's rows and on
    2^norm_log2_rows rows of the same width (HBM-bound: x read and y written
    once, 4 B per element in bf16)."""
    sp = wl.spec
    n, d, v = sp.n, sp.d, sp.v
    x, gamma = workloads.pre_norm(n, d, seed=2, device="cuda")
    flops = 2.0 * n * d * v
    out = {"temperature": EX_TAU, "tokens": n, "hidden": d, "vocab": v}
    for key, kw in (("plain", {}),
                    ("tau_entropy", dict(temperature=EX_TAU, entropy=True)),
                    ("tau_entropy_norm", dict(temperature=EX_TAU, entropy=True, norm_gamma=gamma,
                                              norm_eps=NORM_EPS))):
        rows = x if "norm_gamma" in kw else wl.h
        ws = torch.empty(tim.logprob_ex_workspace_bytes(
            n, d, v, tim.TIM_BF16, temperature=kw.get("temperature", 1.0),
            norm="norm_gamma" in kw, entropy=kw.get("entropy", False)),
            dtype=torch.uint8, device="cuda")
        fn = lambda: tim.tim_logprob_forward_ex(rows, wl.w, wl.ids, workspace=ws, **kw)
        ms = time_calls(fn, torch, np, reps=5, warm=1)
        tf = flops / (ms / 1e3) / 1e12
        out[key] = {"ms": ms, "achieved_TFLOPs": tf, "frac": tf / PEAK_BF16_TFLOPS}
        log(f"scoring {key}: {ms:.3f} ms, {tf:.0f} TFLOP/s ({tf / PEAK_BF16_TFLOPS:.1%})")
        del ws
    y = torch.empty_like(x)
    us = time_calls(lambda: tim.tim_rmsnorm(x, gamma, eps=NORM_EPS, out=y), torch, np,
                    reps=20) * 1e3
    algo = 4 * n * d + 2 * d
    out["rmsnorm_workload"] = {"rows": n, "us": us, "algorithmic_bytes": algo,
                               "achieved_GBs": algo / (us / 1e6) / 1e9}
    del x, y
    torch.cuda.empty_cache()
    nb = 1 << norm_log2_rows
    xb, gb = workloads.pre_norm(nb, d, seed=3, device="cuda")
    yb = torch.empty_like(xb)
    ms = time_calls(lambda: tim.tim_rmsnorm(xb, gb, eps=NORM_EPS, out=yb), torch, np, reps=10)
    algo = 4 * nb * d + 2 * d
    gbs = algo / (ms / 1e3) / 1e9
    out["rmsnorm_scale"] = {"rows": nb, "hidden": d, "ms": ms, "algorithmic_bytes": algo,
                            "achieved_GBs": gbs, "peak_GBs": PEAK_HBM_GBS,
                            "frac": gbs / PEAK_HBM_GBS}
    log(f"rmsnorm: {us:.1f} us at {n} rows; {ms:.3f} ms at 2^{norm_log2_rows} rows = "
        f"{gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%} of HBM)")
    del xb, yb, gb
    torch.cuda.empty_cache()
    return out


def ppo_scale(tim, torch, np, log2n):
    """tim_ppo_loss on 2^log2n tokens with every per-token output: 17 bytes
    read (four fp32 inputs and the mask) and 17 written per token."""
    n = 1 << log2n
    g = torch.Generator(device="cuda").manual_seed(12)
    ot = -torch.rand(n, generator=g, device="cuda") * 4
    orr = ot + torch.randn(n, generator=g, device="cuda") * 0.05
    lp = ot + torch.randn(n, generator=g, device="cuda") * 0.3
    adv = torch.randn(n, generator=g, device="cuda")
    mask = (torch.rand(n, generator=g, device="cuda") < 0.9).to(torch.uint8)
    ws = torch.empty(int(tim.load_library().tim_ppo_workspace_bytes(n)), dtype=torch.uint8,
                     device="cuda")
    outs = {k: torch.empty(n, dtype=torch.float32, device="cuda")
            for k in ("loss", "grad", "ratio", "contrib")}
    clipped = torch.empty(n, dtype=torch.uint8, device="cuda")
    lib = tim.load_library()
    tok = tim._PpoTokenOut(*[outs[k].data_ptr() for k in ("loss", "grad", "ratio", "contrib")],
                           clipped.data_ptr())
    batch = torch.empty(len(tim.PPO_FIELDS), dtype=torch.float64, device="cuda")
    import ctypes
    stream = torch.cuda.current_stream().cuda_stream
    # algorithmic bytes: four fp32 inputs and the mask read, four fp32
    # outputs and the clip flag written, the batch vector
    algo = 34 * n + 8 * len(tim.PPO_FIELDS)
    res = {"tokens": n, "algorithmic_bytes": algo, "peak_GBs": PEAK_HBM_GBS}
    # grad_scale 0: the token mean's gradient (a second pass rescales it);
    # > 0: a caller-given normaliser, one pass
    for key, scale in (("mean_grad", 0.0), ("scaled_grad", 1.0 / n)):
        prm = tim._PpoParams(0.2, 0.28, 0, 2.0, scale)

        def fn():
            st = lib.tim_ppo_loss(lp.data_ptr(), ot.data_ptr(), orr.data_ptr(), adv.data_ptr(),
                                  mask.data_ptr(), n, ctypes.byref(prm), ctypes.byref(tok),
                                  batch.data_ptr(), ws.data_ptr(), ws.numel(), stream)
            assert st == tim.TIM_OK
        ms = time_calls(fn, torch, np, reps=5)
        gbs = algo / (ms / 1e3) / 1e9
        log(f"ppo 2^{log2n} ({key}): {ms:.3f} ms, {gbs:.0f} GB/s "
            f"({gbs / PEAK_HBM_GBS:.1%} of HBM)")
        res[key] = {"ms": ms, "achieved_GBs": gbs, "frac": gbs / PEAK_HBM_GBS}
    del ot, orr, lp, adv, mask, outs, clipped, ws
    torch.cuda.empty_cache()
    # the headline figure: the default (mean) call
    res.update({"ms": res["mean_grad"]["ms"], "achieved_GBs": res["mean_grad"]["achieved_GBs"],
                "frac": res["mean_grad"]["frac"]})
    return res


def invariance_cost(tim, wl, torch, np):
    """t(invariant) / t(schedule) - 1 for the forward at several batch sizes,
    against the free schedule (the fastest configuration the library has for
    that N, allowed to depend on N) and against the K-split schedule (an
    N-dependent split with its own merge, at 33..256 tokens).  The schedules
    are timed alternately, 5 rounds of 4 calls each; the median is kept."""
    res = {}
    for b in (1, 7, 64, 256, 1000, 8192):
        h, ids = wl.h[:b], wl.ids[:b]
        t = {}
        for sch in ("invariant", "free", "split_k"):
            ws = torch.empty(tim.logprob_workspace_bytes(b, wl.spec.d, wl.spec.v, tim.TIM_BF16,
                                                         sch), dtype=torch.uint8, device="cuda")
            t[sch] = (ws, [])
        for _ in range(5):
            for sch, (ws, times) in t.items():
                times.append(time_calls(
                    lambda: tim.tim_logprob_forward(h, wl.w, ids, schedule=sch, workspace=ws),
                    torch, np, reps=4, warm=1))
        ms = {sch: float(np.median(times)) for sch, (_, times) in t.items()}
        split_used = 32 < b <= 256
        res[str(b)] = {"invariant_ms": ms["invariant"], "free_ms": ms["free"],
                       "cost": ms["invariant"] / ms["free"] - 1.0,
                       "split_k_ms": ms["split_k"] if split_used else None,
                       "cost_vs_split_k": ms["invariant"] / ms["split_k"] - 1.0 if split_used else None}
        log(f"invariance cost b={b}: invariant {ms['invariant']:.3f} ms, free {ms['free']:.3f} ms "
            f"({ms['invariant'] / ms['free'] - 1:+.1%})"
            + (f", K split {ms['split_k']:.3f} ms ({ms['invariant'] / ms['split_k'] - 1:+.1%})"
               if split_used else ""))
        del t
    return res


def cpu_baseline(wl, np, rows):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload."""
    import oracle
    h = wl.h.cpu()
    w = wl.w.cpu()
    ids = wl.ids.cpu()
    threads = min(oracle.available_cpus(), oracle.MAX_THREADS)
    if rows <= 0:
        # calibrate: one row per thread, then size to ~15 s
        t = time.perf_counter()
        oracle.logprob(h, w, ids, dtype=oracle.BF16, rows=np.arange(threads), nthreads=threads)
        per_round = time.perf_counter() - t
        rows = max(threads, int(15.0 / max(per_round, 1e-3)) * threads)
        rows = min(rows, wl.spec.n)
    sample = np.linspace(0, wl.spec.n - 1, rows).astype(np.int64)
    log(f"cpu baseline: oracle on {rows} rows with {threads} threads")
    t = time.perf_counter()
    _, _, _, used = oracle.logprob(h, w, ids, dtype=oracle.BF16, rows=sample, nthreads=threads)
    t_lp = time.perf_counter() - t
    lt = wl.logp_sampler.cpu()
    lr = wl.logp_rollout.cpu()
    cu = wl.cu_seqlens.cpu()
    t = time.perf_counter()
    oracle.mismatch_stats(lt, lr, None, cu, clip_c=wl.spec.clip_c, seq_lo=wl.spec.seq_lo,
                          seq_hi=wl.spec.seq_hi)
    t_st = time.perf_counter() - t
    per_token = t_lp / rows + t_st / wl.spec.n
    log(f"cpu baseline: {rows / t_lp:.2f} rows/s logprob, stats {t_st * 1e3:.1f} ms")
    host_cores = len(os.sched_getaffinity(0))
    log(f"cpu baseline: {used} oracle threads on a host with {host_cores} cores available "
        f"to this process ({os.cpu_count()} online)")
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": used,
            "host_cores_affinity": host_cores, "host_cpus_online": os.cpu_count(),
            "kind": "oracle",
            "sample": f"{rows} of {wl.spec.n} rows of the workload (fp64 logprob, evenly "
                      f"spaced) + stats over all {wl.spec.n} tokens; full-N time extrapolated "
                      f"from the sample", "logprob_rows_per_s": rows / t_lp,
            "stats_ms_full_n": t_st * 1e3}


if __name__ == "__main__":
    main()
