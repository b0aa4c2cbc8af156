#!/usr/bin/env python3
"""Benchmark of fused exact attention on one MI355X.

Headline: forward + backward of bf16 multi-head attention, B=4, H=8,
head_dim=128, Tq=Tkv=8192, non-causal, reported in TFLOP/s by the probjax
pages' FLOP convention (forward 4*B*H*Tq*Tkv*D, halved for causal; forward +
backward = 3.5x forward) and as a fraction of the bf16 MFMA peak.

One step = attn_fwd followed by the three passes of attn_bwd on the same
synthetic inputs (inputs resident in HBM before the timed region). W warmup
steps, then exactly K timed steps between device synchronisations; HIP events
around every kernel give the per-kernel average durations used for the
roofline of the dominant kernel.

Also reported (outside the main timed region): the causal variant of the same
shape, and the split-KV GQA decode (B=4, 32 query heads over 8 KV heads,
Tq=16, KV cache 16384, head_dim 128) against the HBM roofline, rotating four
distinct K/V caches so that repeated calls cannot be served from the 256 MB
Infinity Cache. The CPU baseline is the float64 oracle timed on this host's
cores on a bounded sample of the headline workload.

Prints one JSON line on stdout; progress goes to stderr.
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

METRIC = "attention fwd+bwd TFLOP/s, bf16 B4 H8 d128 T8192; % of MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_SYMBOLS = {"attn_fwd": "attn_fwd_bf16_kernel",
                  "bwd_dkdv": "attn_dkdv_queue_kernel", "bwd_dq": "attn_dq_pair_kernel",
                  "decode_split": "attn_decode_split_kernel", "decode_combine": "attn_decode_combine_kernel"}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the causal and decode legs")
    ap.add_argument("--decode-calls", type=int, default=200)
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="also time plain bf16 GEMMs through torch (hipBLASLt) as a practical MFMA ceiling")
    ap.add_argument("--fp32-suite", action="store_true", help="time the fp32 grid (batch 4, 8 heads, head_dim 64/128)")
    ap.add_argument("--suites", action="store_true",
                    help="also time the GQA suite (fwd+bwd, native GQA against repeated K/V), the decode suite, a head_dim "
                         "sweep, the head_dim-64 grid and the KV-length case")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of this many MiB (reference dispatch for HBM counters)")
    ap.add_argument("--summarize", nargs=3, metavar=("STATS_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="turn rocprofv3 CSV output (kernel-trace stats, FETCH_SIZE pass, WRITE_SIZE pass) into "
                         "the summaries under profiles/ and exit (no GPU use)")
    ap.add_argument("--summarize-fp32", metavar="STATS_DIR",
                    help="turn a rocprofv3 kernel trace of the fp32 suite into profiles/fp32_grid_kernel_stats.md "
                         "and exit (no GPU use); --profile-command records the command")
    ap.add_argument("--summarize-suites", metavar="BENCH_LOG",
                    help="turn the JSON line of a `bench.py --suites` run (the last line starting with '{' in "
                         "BENCH_LOG) into profiles/suites_and_legs.md and exit (no GPU use); --profile-command "
                         "records the command")
    ap.add_argument("--profile-command", default="", help="kernel-trace command recorded in the summaries")
    ap.add_argument("--counter-command", default="", help="counter-pass command recorded in the summaries")
    ap.add_argument("--mfma-dir", default="", help="with --summarize: rocprofv3 output of a pass with "
                    "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_BUSY_CYCLES GRBM_GUI_ACTIVE")
    ap.add_argument("--mfma-command", default="", help="MFMA counter-pass command recorded in the summaries")
    ap.add_argument("--summarize-stalls", nargs="+", metavar="PMC_DIR",
                    help="turn rocprofv3 --pmc passes over the headline run (issue, wait, co-issue and LDS counters) "
                         "into profiles/fwd_bwd_d128_T8192_issue_counters.md and exit (no GPU use); "
                         "--counter-command records the command of each pass")
    return ap.parse_args()


def source_digest():
    """Digest of the HIP sources: stored counter readings are only valid for the kernels they measured."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "forward_backward_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, path: str = ""):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None if stale/missing."""
    path = path or os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("kernels", {}).get(kernel)
    if not entry or rec.get("source_digest") != source_digest():
        return None
    return entry.get("bytes_per_launch")


def _short_name(kernel_name):
    import re
    k = kernel_name.replace("void ", "").replace("attn::(anonymous namespace)::", "")
    return re.sub(r"\(.*", "", k)


def _read_counter_csv(directory, counter, first_leg=0):
    """Per-kernel list of per-dispatch values of `counter` from a rocprofv3 --pmc CSV.

    With first_leg > 0 only the first `first_leg` dispatches of each non-decode
    kernel count (bench.py runs the headline leg first; the causal, window and
    other legs launch the same kernels on other workloads). Decode kernels
    only ever run the one decode workload, so all their dispatches count.
    """
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (_short_name(r["Kernel_Name"]), int(r["Dispatch_Id"]), r["Grid_Size"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    by_name = {}
    for (name, did, grid), v in per.items():
        by_name.setdefault(name, []).append((did, grid, v))
    for ds in by_name.values():
        ds.sort()
    # The headline leg ends where the first attention kernel of the run (the
    # forward) is dispatched for the first_leg + 1-th time.
    bound = None
    if first_leg:
        attn = [(ds[0][0], name) for name, ds in by_name.items()
                if name.startswith("attn") and not name.startswith("attn_decode")]
        if attn:
            lead = by_name[min(attn)[1]]
            bound = lead[first_leg][0] if len(lead) > first_leg else None
    out = {}
    for name, ds in by_name.items():
        if bound is not None and not name.startswith("attn_decode") and "copyBuffer" not in name:
            ds = [d for d in ds if d[0] < bound]
        for _, grid, v in ds:
            out.setdefault((name, grid), []).append(v)
    return out


def summarize(stats_dir, fetch_dir, write_dir, command, counter_command, out_dir=""):
    """Write profiles/ summaries (or into out_dir) from rocprofv3 output (runs on any host)."""
    import csv
    import glob

    prof = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    rows = []
    for path in glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            rows.append((_short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]), float(r["TotalDurationNs"]),
                         float(r["MinNs"]), float(r["MaxNs"])))
    rows.sort(key=lambda x: -x[3])
    lines = ["# Kernel durations: attention fwd+bwd B4 H8 d128 T8192 (+ causal and GQA decode legs)", "",
             "Produced by:", "", "```", command or "(command not recorded)", "```", "",
             "| kernel | calls | average us | min us | max us | total ms |", "|---|---|---|---|---|---|"]
    for name, calls, avg, tot, mn, mx in rows:
        if not name.startswith("attn"):
            continue
        lines.append(f"| `{name}` | {calls} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | {tot / 1e6:.3f} |")
    # Per-leg averages from the dispatch trace: bench.py runs the non-causal
    # headline leg first (warmup + steps dispatches of each kernel), then the
    # causal leg (1 warmup + steps).
    import re as _re
    w = int((_re.search(r"--warmup (\d+)", command or "") or [None, 3])[1])
    k = int((_re.search(r"--steps (\d+)", command or "") or [None, 20])[1])
    per_kernel = {}
    for path in glob.glob(os.path.join(stats_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            name = _short_name(r["Kernel_Name"])
            if name.startswith("attn"):
                per_kernel.setdefault(name, []).append(
                    (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    lines += ["", "Per leg, from the dispatch trace (the headline non-causal leg runs first: "
              f"{w} warmup + {k} timed steps; then the causal leg):", "",
              "| kernel | headline leg: dispatches | headline leg: average us (timed steps) | causal leg: average us |",
              "|---|---|---|---|"]
    for ds in per_kernel.values():
        ds.sort()
    # Kernels first launched after the headline leg (short-sequence legs and
    # the like) belong to other workloads.
    lead = min((ds[0][0], name) for name, ds in per_kernel.items()) if per_kernel else None
    leg_end = per_kernel[lead[1]][w + k][0] if lead and len(per_kernel[lead[1]]) > w + k else None
    for name, ds in sorted(per_kernel.items()):
        if name.startswith("attn_decode") or (leg_end is not None and ds[0][0] >= leg_end):
            continue
        head = [d for _, d in ds[:w + k]]
        timed = head[w:] if len(head) > w else head
        rest = [d for _, d in ds[w + k:w + k + 1 + k]][1:]
        lines.append(f"| `{name}` | {len(head)} | {sum(timed) / max(len(timed), 1) / 1e3:.2f} | "
                     f"{(sum(rest) / len(rest) / 1e3) if rest else float('nan'):.2f} |")
    with open(os.path.join(prof, "fwd_bwd_d128_T8192_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    cw = int((_re.search(r"--warmup (\d+)", counter_command or "") or [None, 3])[1])
    ck = int((_re.search(r"--steps (\d+)", counter_command or "") or [None, 20])[1])
    fetch = _read_counter_csv(fetch_dir, "FETCH_SIZE", cw + ck)
    write = _read_counter_csv(write_dir, "WRITE_SIZE", cw + ck)
    copy_f = [v for (n, g), vs in fetch.items() if "copyBuffer" in n for v in vs]
    copy_w = [v for (n, g), vs in write.items() if "copyBuffer" in n for v in vs]
    copy_kib = None
    # The calibration dispatch is the largest plain copy in the run.
    if copy_w:
        copy_kib = max(copy_w)
    f_factor = copy_kib / max(copy_f) if copy_f and copy_kib else None
    w_factor = 1.0 if copy_kib else None
    lines = ["# HBM traffic per dispatch: attention fwd+bwd B4 H8 d128 T8192 non-causal, and GQA decode", "",
             "Two rocprofv3 counter passes of the command below, one with FETCH_SIZE, one with WRITE_SIZE (KiB "
             "per dispatch), each scaled by what the counter reads for a plain device copy of known size run in "
             "the same process (`--copy-calibration 256`: 256 MiB read, 256 MiB written). The fwd/bwd rows are "
             "the headline leg's dispatches (the run's first leg); the decode rows are every dispatch of the "
             "decode leg (batch 4, 16 query rows, 16384-key caches, 32 query heads over 8 KV heads).", "",
             "```", counter_command or "", "```", "",
             f"Copy calibration: WRITE_SIZE {copy_kib} KiB for 262144 KiB written (factor {w_factor}); "
             f"FETCH_SIZE {max(copy_f) if copy_f else None} KiB for 262144 KiB read (factor {f_factor}).", "",
             "| kernel | grid | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM MiB per launch |", "|---|---|---|---|---|"]
    traffic = {}
    for (name, grid), fv in sorted(fetch.items()):
        if not name.startswith("attn"):
            continue
        wv = write.get((name, grid), [0.0])
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        total = None
        if f_factor:
            total = (fk * f_factor + wk * w_factor) * 1024
            base = name.split("<")[0]
            if base not in traffic or total > traffic[base]:
                traffic[base] = total
        lines.append(f"| `{name}` | {grid} | {fk:.0f} | {wk:.0f} | "
                     f"{'' if total is None else f'{total / 2**20:.1f}'} |")
    with open(os.path.join(prof, "fwd_bwd_d128_T8192_hbm_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(prof, "hbm_traffic.json"), "w") as f:
        json.dump({"source_digest": source_digest(), "command": counter_command,
                   "kernels": {k: {"bytes_per_launch": round(v)} for k, v in traffic.items()}}, f, indent=1)
    print(f"wrote summaries under {prof}")


def summarize_fp32(stats_dir, command, out_dir=""):
    """Per-kernel, per-grid durations of a kernel trace of the fp32 suite (B4 H8, head_dim 64/128)."""
    import csv
    import glob
    from forward_backward_amd.inputs import workload_cases
    from forward_backward_amd.metrics import attention_flops

    runs = {}
    for path in glob.glob(os.path.join(stats_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            name = _short_name(r["Kernel_Name"])
            if "f32_kernel" not in name:
                continue
            grid = int(r["Grid_Size_X"]) if "Grid_Size_X" in r else int(r["Grid_Size"])
            runs.setdefault((name, grid), []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    # Grid (threads) of each kernel per case, to name the shape and price the launch.
    shapes = {}
    for c in workload_cases(8):
        fwd_f = attention_flops(c.B, c.Hq, c.Tq, c.Tkv, c.D, c.causal, "fwd")
        nq, nk = -(-c.Tq // 128), -(-c.Tkv // 128)
        for kern, grid, fl in ((f"attn_fwd_f32_kernel<{c.D}>", 256 * nq * c.Hq * c.B, fwd_f),
                               (f"attn_dq_f32_kernel<{c.D}>", 256 * nq * c.Hq * c.B, 1.5 * fwd_f),
                               (f"attn_dkdv_f32_kernel<{c.D}>", 256 * nk * c.Hkv * c.B, 2 * fwd_f)):
            shapes.setdefault((kern, grid), []).append((c, fl))
    lines = ["# fp32 kernels on the fp32 matrix cores: the fp32 grid (B4 H8, head_dim 64/128)", "",
             "rocprofv3 kernel trace of the command below (each shape timed non-causal, then causal; a grid "
             "covers both). TFLOP/s = the launch's algorithmic FLOPs (forward 4, dK/dV 8, dQ 6 x B H Tq Tkv D, "
             "halved when causal) / median duration; peak 157.3 TFLOP/s (fp32 matrix).", "",
             "```", command or "(command not recorded)", "```", "",
             "| kernel | grid (threads) | shape | dispatches | median us | TFLOP/s | of fp32 peak |",
             "|---|---|---|---|---|---|---|"]
    for (name, grid), ds in sorted(runs.items()):
        cases = shapes.get((name, grid), [])
        ds = [d for _, d in sorted(ds)]
        # Both cases of a shape share the grid; the suite runs the non-causal one first, with as many
        # dispatches as the causal one.
        halves = [("full", ds[:len(ds) // 2]), ("causal", ds[len(ds) // 2:])] if len(cases) == 2 else [("", ds)]
        for tag, part in halves:
            if not part:
                continue
            med = sorted(part)[len(part) // 2]
            case = next((c for c, _ in cases if (tag == "causal") == c.causal), None) if cases else None
            fl = next((f for c, f in cases if case is not None and c is case), None)
            tf = f"{fl / (med * 1e-9) / 1e12:.1f}" if fl else ""
            frac = f"{fl / (med * 1e-9) / 1e12 / 157.3:.0%}" if fl else ""
            lines.append(f"| `{name}` | {grid} | {case.name if case else '?'} | {len(part)} | {med / 1e3:.1f} | "
                         f"{tf} | {frac} |")
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), "fp32_grid_kernel_stats.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {path}")


def summarize_mfma(stats_dir, mfma_dir, command, profile_command, out_dir=""):
    """MFMA utilisation per kernel at the clock the chip actually ran.

    SQ_VALU_MFMA_BUSY_CYCLES sums the busy cycles of every SIMD's matrix unit;
    GRBM_GUI_ACTIVE sums the GPU's active cycles over the 8 XCDs. Dividing the
    latter by 8 and by the kernel's duration (kernel-trace average of the same
    leg) gives the clock; busy / (cycles per XCD * 1024 SIMDs) is the fraction
    of the matrix units' time spent on MFMAs, independent of the clock.
    """
    import csv
    import glob
    import re
    w = int((re.search(r"--warmup (\d+)", profile_command or "") or [None, 3])[1])
    k = int((re.search(r"--steps (\d+)", profile_command or "") or [None, 20])[1])
    busy = _read_counter_csv(mfma_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    insts = _read_counter_csv(mfma_dir, "SQ_INSTS_MFMA")
    grbm = _read_counter_csv(mfma_dir, "GRBM_GUI_ACTIVE")
    durations = {}
    for path in glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            durations[_short_name(r["Name"])] = float(r["AverageNs"])
    # Durations of the headline leg (the kernel-trace average mixes in the causal leg).
    trace = {}
    for path in glob.glob(os.path.join(stats_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            trace.setdefault(_short_name(r["Kernel_Name"]), []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    lines = ["# MFMA utilisation: attention fwd+bwd B4 H8 d128 T8192, non-causal", "",
             "One rocprofv3 counter pass (SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA, SQ_BUSY_CYCLES, GRBM_GUI_ACTIVE) "
             "of the command below. GRBM_GUI_ACTIVE sums active cycles over the 8 XCDs; divided by 8 and by the "
             "kernel's headline-leg duration from the kernel trace it gives the clock the chip ran at. "
             "`MFMA busy` = SQ_VALU_MFMA_BUSY_CYCLES / (cycles per XCD x 1024 SIMDs): the fraction of the matrix "
             "units' time spent on MFMAs at that clock (the published peak assumes 2.4 GHz).", "",
             "```", command or "", "```", "",
             "| kernel | MFMA instructions | busy cycles per MFMA | cycles per XCD | duration us | clock GHz | "
             "MFMA busy |", "|---|---|---|---|---|---|---|"]
    for (name, grid), bv in sorted(busy.items()):
        if not name.startswith("attn") or name not in trace:
            continue
        b = sum(bv) / len(bv)
        if b == 0:
            continue
        n = sum(insts.get((name, grid), [0.0])) / max(len(insts.get((name, grid), [1])), 1)
        g = sum(grbm.get((name, grid), [0.0])) / max(len(grbm.get((name, grid), [1])), 1)
        head = sorted(d for _, d in sorted(trace[name])[w:w + k])  # timed steps of the headline leg
        dur = head[len(head) // 2] / 1e3  # median, us
        cyc = g / 8
        lines.append(f"| `{name}` | {n:.4g} | {b / max(n, 1):.1f} | {cyc:.4g} | {dur:.1f} | "
                     f"{cyc / (dur * 1e3):.2f} | {b / (cyc * 1024):.1%} |")
    with open(os.path.join(out_dir or os.path.join(ROOT, "profiles"), "fwd_bwd_d128_T8192_mfma_util.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote MFMA utilisation summary")


def device_tensors(case, seed=0, with_do=True):
    import numpy as np
    import torch
    from forward_backward_amd import inputs as I

    host = I.make_inputs(case, seed=seed, with_do=with_do)
    dev = {}
    for k, v in host.items():
        if v is None:
            dev[k] = None
        elif k == "kv_lens":
            dev[k] = torch.from_numpy(v).cuda()
        else:
            dev[k] = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).cuda()
    return host, dev


def quartiles(xs):
    """Median, first and third quartile (linear interpolation), min and max."""
    v = sorted(xs)
    n = len(v)

    def q(f):
        x = f * (n - 1)
        i = int(x)
        return v[i] if i + 1 >= n else v[i] + (x - i) * (v[i + 1] - v[i])

    return {"median": round(q(0.5), 4), "q1": round(q(0.25), 4), "q3": round(q(0.75), 4),
            "min": round(v[0], 4), "max": round(v[-1], 4)}


def time_train_steps(case, steps, warmup, spread=False):
    """K timed fwd+bwd steps; returns (ms_per_step, {kernel: avg_ms}) and, with
    spread, the median and quartiles of the K per-step and per-kernel times."""
    import torch
    from forward_backward_amd import attn

    _, d = device_tensors(case)
    q, k, v, do = d["q"], d["k"], d["v"], d["do"]
    kv = d["kv_lens"]
    o = torch.empty_like(q)
    lse = torch.empty((case.B, case.Hq, case.Tq), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = attn.bwd_workspace(q, k, case.causal, kv)
    kw = dict(scale=case.scale, causal=case.causal, kv_lens=kv, window=case.window)

    # The passes attn_bwd runs, in its order: dQ with the preprocess outputs
    # (D formed in the dQ kernel at bf16 head_dim 64/128), then dK/dV.
    def step(ev=None):
        attn.fwd(q, k, v, out=o, lse=lse, **kw)
        if ev: ev[1].record()
        attn.bwd_dq_and_preprocess(q, k, v, o, lse, do, ws, dq, **kw)
        if ev: ev[2].record()
        attn.bwd_dkdv(q, k, v, lse, do, ws, dk, dv, **kw)
        if ev: ev[3].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        evs[i][0].record()
        step(evs[i])
    torch.cuda.synchronize()
    total = evs[0][0].elapsed_time(evs[-1][3])
    names = ["attn_fwd", "bwd_dq", "bwd_dkdv"]
    per = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j, n in enumerate(names)}
    if not torch.isfinite(dq.float()).all() or not torch.isfinite(o.float()).all():
        raise RuntimeError("non-finite outputs in the benchmark step")
    if not spread:
        return total / steps, per
    dist = {"step_ms": quartiles([e[0].elapsed_time(e[3]) for e in evs]),
            "per_kernel_ms": {n: quartiles([e[j].elapsed_time(e[j + 1]) for e in evs]) for j, n in enumerate(names)}}
    return total / steps, per, dist


def time_decode(case, calls, sets=4):
    """Average ms per attn_decode call, rotating `sets` distinct K/V caches.

    Returns (graph, eager, same_cache, kv_lens): `graph` replays a HIP graph
    of `calls` captured calls (device time without the host's per-call
    launch cost), `eager` issues the calls from Python one by one, and
    `same_cache` repeats one cache (warm in the chip's caches).
    """
    import torch
    from forward_backward_amd import attn

    host, d0 = device_tensors(case, seed=0, with_do=False)
    caches = [(d0["k"], d0["v"])]
    for s in range(1, sets):
        _, ds = device_tensors(case, seed=s, with_do=False)
        caches.append((ds["k"], ds["v"]))
    q, kv = d0["q"], d0["kv_lens"]
    ws = attn.decode_workspace(q, caches[0][0])  # one workspace for every call
    for i in range(4):
        attn.decode(q, *caches[i % sets], kv_lens=kv, scale=case.scale, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / calls

    def eager():
        for i in range(calls):
            attn.decode(q, *caches[i % sets], kv_lens=kv, scale=case.scale, workspace=ws)

    def same():
        for i in range(calls):
            attn.decode(q, *caches[0], kv_lens=kv, scale=case.scale, workspace=ws)

    cold = timed(eager)
    warm = timed(same)
    mem = decode_memory(q, caches[0], kv, case.scale)
    # Outputs and workspaces allocated during capture live in the graph's
    # memory pool for as long as the graph object does.
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            eager()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    replay = min(timed(graph.replay) for _ in range(3))
    del graph
    return replay, cold, warm, [int(x) for x in host["kv_lens"]], mem


def decode_memory(q, cache, kv, scale):
    """Workspace bytes, output bytes (O and LSE) and the device peak beyond the
    inputs of one attn_decode call that allocates its own outputs and workspace."""
    import ctypes
    import torch
    from forward_backward_amd import attn

    B, Tq, Hq, D = q.shape
    _, Tkv, Hkv, _ = cache[0].shape
    p = attn.make_params(B, Tq, Tkv, Hq, Hkv, D)
    ws = int(attn.lib().attn_decode_workspace_size(ctypes.byref(p), 0))
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    o, lse = attn.decode(q, *cache, kv_lens=kv, scale=scale)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    out = o.numel() * o.element_size() + lse.numel() * lse.element_size()
    return {"workspace_bytes": ws, "output_bytes": int(out), "device_peak_bytes": int(peak),
            "device_peak": "beyond the resident inputs; torch's caching allocator rounds each block up"}


def gemm_ceiling():
    """bf16 GEMM rate of the vendor library through torch: a practical MFMA ceiling for this chip."""
    import torch
    rows = []
    for m, n, k in ((8192, 8192, 8192), (16384, 16384, 8192)):
        a = device_normal((m, k), 1)
        b = device_normal((k, n), 2)
        for _ in range(5):
            c = a @ b
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        rows.append({"m": m, "n": n, "k": k, "ms": round(ms, 4), "tflops": round(2 * m * n * k / (ms * 1e-3) / 1e12, 1)})
        log(f"  gemm {m}x{n}x{k}: {ms:.3f} ms, {rows[-1]['tflops']} TFLOP/s")
        del a, b, c
    return rows


def device_normal(shape, seed, dtype="bf16"):
    """Seeded N(0,1) tensor drawn on the device (timing legs only; no oracle reads it)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def _time_steps(q, k, v, do, case, steps, warmup):
    """ms per fwd+bwd step on given tensors; returns (ms, peak bytes allocated beyond the inputs)."""
    import torch
    from forward_backward_amd import attn

    kw = dict(scale=case.scale, causal=case.causal)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()

    def step():
        o, lse = attn.fwd(q, k, v, **kw)
        return attn.bwd(q, k, v, o, lse, do, **kw)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, peak


def gqa_suite(steps):
    """The pages' GQA suite: 32 query heads over 8 KV heads, head_dim 128, batch 1, Lq = Lkv = T.

    Times fwd+bwd with native GQA (query head h reads KV head h // G) and the
    same problem run as plain multi-head attention on K/V repeated G times
    (dK/dV summed over each group afterwards), and reports the peak device
    memory of each beyond the inputs.
    """
    import torch
    from forward_backward_amd.inputs import workload_cases
    from forward_backward_amd.metrics import attention_flops

    rows = []
    for case in workload_cases(5):
        G = case.Hq // case.Hkv
        q = device_normal((case.B, case.Tq, case.Hq, case.D), 1)
        k = device_normal((case.B, case.Tkv, case.Hkv, case.D), 2)
        v = device_normal((case.B, case.Tkv, case.Hkv, case.D), 3)
        do = device_normal((case.B, case.Tq, case.Hq, case.D), 4)
        ms, peak = _time_steps(q, k, v, do, case, steps, 2)

        def repeated():
            kr = k.repeat_interleave(G, dim=2)
            vr = v.repeat_interleave(G, dim=2)
            from forward_backward_amd import attn
            o, lse = attn.fwd(q, kr, vr, scale=case.scale)
            dq, dkr, dvr = attn.bwd(q, kr, vr, o, lse, do, scale=case.scale)
            sh = (case.B, case.Tkv, case.Hkv, G, case.D)
            return dq, dkr.view(sh).float().sum(3).to(torch.bfloat16), dvr.view(sh).float().sum(3).to(torch.bfloat16)

        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        repeated()
        torch.cuda.synchronize()
        peak_rep = torch.cuda.max_memory_allocated() - base
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            repeated()
        e1.record()
        torch.cuda.synchronize()
        ms_rep = e0.elapsed_time(e1) / steps
        fl = attention_flops(case.B, case.Hq, case.Tq, case.Tkv, case.D, case.causal, "fwd_bwd")
        row = {"T": case.Tq, "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
               "peak_mb": round(peak / 2**20, 1), "repeated_ms": round(ms_rep, 4),
               "repeated_peak_mb": round(peak_rep / 2**20, 1)}
        rows.append(row)
        log(f"  gqa T{case.Tq}: {ms:.3f} ms ({row['tflops']} TFLOP/s), peak {row['peak_mb']} MB; "
            f"repeated K/V {ms_rep:.3f} ms, peak {row['repeated_peak_mb']} MB")
        del q, k, v, do
    return {"shape": "bf16 B1 Hq32 Hkv8 d128 Lq=Lkv=T non-causal, fwd+bwd", "rows": rows}


def headdim_sweep(steps):
    """fwd+bwd at B4 H8 T4096 (non-causal) for head_dim 32, 64, 128 and 256 (bf16)."""
    from forward_backward_amd.inputs import Case
    from forward_backward_amd.metrics import attention_flops

    rows = []
    for d in (32, 64, 128, 256):
        case = Case(f"bf16_B4_H8_T4096_d{d}", 4, 4096, 4096, 8, 8, d, "bf16", False, workload_id=8)
        q = device_normal((case.B, case.Tq, case.Hq, d), 1)
        k = device_normal((case.B, case.Tkv, case.Hkv, d), 2)
        v = device_normal((case.B, case.Tkv, case.Hkv, d), 3)
        do = device_normal((case.B, case.Tq, case.Hq, d), 4)
        ms, _ = _time_steps(q, k, v, do, case, steps, 2)
        fl = attention_flops(case.B, case.Hq, case.Tq, case.Tkv, d, False, "fwd_bwd")
        rows.append({"D": d, "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1)})
        log(f"  d{d}: {ms:.3f} ms ({rows[-1]['tflops']} TFLOP/s)")
        del q, k, v, do
    return {"shape": "bf16 B4 H8 T4096 non-causal, fwd+bwd", "rows": rows}


def _fwd_ms(q, k, v, kw, n):
    import torch
    from forward_backward_amd import attn
    for _ in range(2):
        attn.fwd(q, k, v, **kw)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        attn.fwd(q, k, v, **kw)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _step_ms(q, k, v, do, kw, n):
    import torch
    from forward_backward_amd import attn

    def step():
        o, lse = attn.fwd(q, k, v, **kw)
        return attn.bwd(q, k, v, o, lse, do, **kw)
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        step()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def short_and_kvlen_legs(n):
    """The head_dim-64 grid's lengths up to 1024 (fwd and fwd+bwd, causal and not) and the KV-length
    workload (fwd+bwd, TFLOP/s over the nominal FLOPs and over the keys inside the lengths)."""
    import torch
    from forward_backward_amd.inputs import make_inputs, workload_cases
    from forward_backward_amd.metrics import attention_flops, effective_flops

    rows = []
    for case in workload_cases(1):
        if case.Tq > 1024:
            continue
        q = device_normal((case.B, case.Tq, case.Hq, case.D), 1)
        k = device_normal((case.B, case.Tkv, case.Hkv, case.D), 2)
        v = device_normal((case.B, case.Tkv, case.Hkv, case.D), 3)
        do = device_normal((case.B, case.Tq, case.Hq, case.D), 4)
        kw = dict(scale=case.scale, causal=case.causal)
        f_ms, fb_ms = _fwd_ms(q, k, v, kw, n), _step_ms(q, k, v, do, kw, n)
        ffl = attention_flops(case.B, case.Hq, case.Tq, case.Tkv, case.D, case.causal, "fwd")
        fbfl = attention_flops(case.B, case.Hq, case.Tq, case.Tkv, case.D, case.causal, "fwd_bwd")
        rows.append({"case": case.name, "fwd_us": round(f_ms * 1e3, 2), "fwd_tflops": round(ffl / (f_ms * 1e-3) / 1e12, 1),
                     "fwd_bwd_us": round(fb_ms * 1e3, 2),
                     "fwd_bwd_tflops": round(fbfl / (fb_ms * 1e-3) / 1e12, 1)})
        log(f"  {case.name}: fwd {f_ms * 1e3:.1f} us, fwd+bwd {fb_ms * 1e3:.1f} us")
        del q, k, v, do
    (case,) = workload_cases(3)
    lens = [int(x) for x in make_inputs(case, with_do=False)["kv_lens"]]
    q = device_normal((case.B, case.Tq, case.Hq, case.D), 1)
    k = device_normal((case.B, case.Tkv, case.Hkv, case.D), 2)
    v = device_normal((case.B, case.Tkv, case.Hkv, case.D), 3)
    do = device_normal((case.B, case.Tq, case.Hq, case.D), 4)
    kw = dict(scale=case.scale, causal=False, kv_lens=torch.tensor(lens, dtype=torch.int32, device=q.device))
    fb_ms = _step_ms(q, k, v, do, kw, n)
    nominal = attention_flops(case.B, case.Hq, case.Tq, case.Tkv, case.D, False, "fwd_bwd")
    eff = effective_flops(case.Hq, case.Tq, lens, case.D, "fwd_bwd")
    kvlen = {"workload": case.name, "kv_lens": lens, "fwd_bwd_ms": round(fb_ms, 4),
             "nominal_tflops": round(nominal / (fb_ms * 1e-3) / 1e12, 1),
             "effective_tflops": round(eff / (fb_ms * 1e-3) / 1e12, 1),
             "effective_frac": round(eff / (fb_ms * 1e-3) / 1e12 / 2516.6, 4)}
    log(f"  {case.name}: fwd+bwd {fb_ms:.3f} ms, {kvlen['effective_tflops']} TFLOP/s effective")
    return {"shape": "bf16 B4 H8 d64, T <= 1024", "rows": rows}, kvlen


def memory_suite():
    """The pages' memory figures ("Attention performance", section "Memory"): the device peak of one
    fwd+bwd call (bf16, head_dim 64, batch 4, 8 heads, non-causal) by length, up to 65536 (the length
    the pages' search stopped at), and the bytes kept for the backward (O and LSE; batch 2, 8 heads,
    head_dim 64)."""
    import torch
    from forward_backward_amd import attn

    peak_rows, res_rows = [], []
    for T in (1024, 4096, 16384, 65536):
        q = device_normal((4, T, 8, 64), 1)
        k = device_normal((4, T, 8, 64), 2)
        v = device_normal((4, T, 8, 64), 3)
        do = device_normal((4, T, 8, 64), 4)
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        o, lse = attn.fwd(q, k, v)
        dq, dk, dv = attn.bwd(q, k, v, o, lse, do)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        peak_rows.append({"T": T, "ran": True, "device_peak_mb": round(peak / 2**20, 2),
                          "inputs_mb": round(4 * q.numel() * 2 / 2**20, 1)})
        log(f"  fwd+bwd B4 H8 d64 T{T}: peak {peak / 2**20:.1f} MB beyond the inputs")
        del q, k, v, do, o, lse, dq, dk, dv
        q = device_normal((2, T, 8, 64), 1)
        k = device_normal((2, T, 8, 64), 2)
        o, lse = attn.fwd(q, k, k)
        res = o.numel() * o.element_size() + lse.numel() * lse.element_size()
        res_rows.append({"T": T, "residual_mb": round(res / 2**20, 3), "kept": "O (bf16) and LSE (fp32)"})
        del q, k, o, lse
    return {"device_peak": {"shape": "bf16 B4 H8 d64 non-causal, one fwd+bwd call, beyond q/k/v/dO",
                            "largest_T_run": 65536, "rows": peak_rows},
            "residuals": {"shape": "bf16 B2 H8 d64, bytes kept for the backward", "rows": res_rows}}


def config_grid(steps):
    """The pages' head_dim-64 grid (bf16 B4 H8 d64, T in {512, 1024, 2048, 600, 1500, 3000}, causal and
    not; fwd and fwd+bwd) and the KV-length case (bf16 B4 H8 d128 T4096, kv_len {1, 777, 2500, 4096},
    fwd+bwd, TFLOP/s over both the nominal and the effective FLOPs, i.e. the keys inside each length)."""
    import torch
    from forward_backward_amd import attn
    from forward_backward_amd.inputs import make_inputs, workload_cases
    from forward_backward_amd.metrics import attention_flops, effective_flops

    def fwd_ms(q, k, v, kw, n):
        for _ in range(2):
            attn.fwd(q, k, v, **kw)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            attn.fwd(q, k, v, **kw)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def step_ms(q, k, v, do, kw, n):
        def step():
            o, lse = attn.fwd(q, k, v, **kw)
            return attn.bwd(q, k, v, o, lse, do, **kw)
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            step()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    n = max(steps, 20)
    rows = []
    for case in workload_cases(1):
        q = device_normal((case.B, case.Tq, case.Hq, case.D), 1)
        k = device_normal((case.B, case.Tkv, case.Hkv, case.D), 2)
        v = device_normal((case.B, case.Tkv, case.Hkv, case.D), 3)
        do = device_normal((case.B, case.Tq, case.Hq, case.D), 4)
        kw = dict(scale=case.scale, causal=case.causal)
        f_ms, fb_ms = fwd_ms(q, k, v, kw, n), step_ms(q, k, v, do, kw, n)
        ffl = attention_flops(case.B, case.Hq, case.Tq, case.Tkv, case.D, case.causal, "fwd")
        fbfl = attention_flops(case.B, case.Hq, case.Tq, case.Tkv, case.D, case.causal, "fwd_bwd")
        rows.append({"case": case.name, "fwd_ms": round(f_ms, 4), "fwd_tflops": round(ffl / (f_ms * 1e-3) / 1e12, 1),
                     "fwd_bwd_ms": round(fb_ms, 4), "fwd_bwd_tflops": round(fbfl / (fb_ms * 1e-3) / 1e12, 1)})
        log(f"  {case.name}: fwd {f_ms * 1e3:.1f} us ({rows[-1]['fwd_tflops']} TFLOP/s), fwd+bwd {fb_ms * 1e3:.1f} us "
            f"({rows[-1]['fwd_bwd_tflops']} TFLOP/s)")
        del q, k, v, do
    (case,) = workload_cases(3)
    lens = [int(x) for x in make_inputs(case, with_do=False)["kv_lens"]]
    q = device_normal((case.B, case.Tq, case.Hq, case.D), 1)
    k = device_normal((case.B, case.Tkv, case.Hkv, case.D), 2)
    v = device_normal((case.B, case.Tkv, case.Hkv, case.D), 3)
    do = device_normal((case.B, case.Tq, case.Hq, case.D), 4)
    kl = torch.tensor(lens, dtype=torch.int32, device=q.device)
    kw = dict(scale=case.scale, causal=False, kv_lens=kl)
    fb_ms = step_ms(q, k, v, do, kw, n)
    nominal = attention_flops(case.B, case.Hq, case.Tq, case.Tkv, case.D, False, "fwd_bwd")
    eff = effective_flops(case.Hq, case.Tq, lens, case.D, "fwd_bwd")
    kvlen = {"case": case.name, "kv_lens": lens, "fwd_bwd_ms": round(fb_ms, 4),
             "nominal_tflops": round(nominal / (fb_ms * 1e-3) / 1e12, 1),
             "effective_tflops": round(eff / (fb_ms * 1e-3) / 1e12, 1)}
    log(f"  {case.name} kv_lens {lens}: fwd+bwd {fb_ms:.3f} ms, {kvlen['effective_tflops']} TFLOP/s effective "
        f"({kvlen['nominal_tflops']} nominal)")
    return {"head_dim64_grid": {"shape": "bf16 B4 H8 d64", "rows": rows}, "kv_len": kvlen}


FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix peak


def fp32_suite(steps):
    """The pages' fp32 grid: batch 4, 8 heads, head_dim 64 and 128, T = 1024 ... 8192, fwd and fwd+bwd."""
    import torch
    from forward_backward_amd import attn
    from forward_backward_amd.inputs import workload_cases
    from forward_backward_amd.metrics import attention_flops

    rows = []
    for case in workload_cases(8):
        q = device_normal((case.B, case.Tq, case.Hq, case.D), 1, "fp32")
        k = device_normal((case.B, case.Tkv, case.Hkv, case.D), 2, "fp32")
        v = device_normal((case.B, case.Tkv, case.Hkv, case.D), 3, "fp32")
        do = device_normal((case.B, case.Tq, case.Hq, case.D), 4, "fp32")
        ms, _ = _time_steps(q, k, v, do, case, steps, 2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(2):
            attn.fwd(q, k, v, scale=case.scale, causal=case.causal)
        e0.record()
        for _ in range(steps):
            attn.fwd(q, k, v, scale=case.scale, causal=case.causal)
        e1.record()
        torch.cuda.synchronize()
        fwd_ms = e0.elapsed_time(e1) / steps
        fl = attention_flops(case.B, case.Hq, case.Tq, case.Tkv, case.D, case.causal, "fwd_bwd")
        ffl = attention_flops(case.B, case.Hq, case.Tq, case.Tkv, case.D, case.causal, "fwd")
        tf, ftf = fl / (ms * 1e-3) / 1e12, ffl / (fwd_ms * 1e-3) / 1e12
        rows.append({"case": case.name, "fwd_ms": round(fwd_ms, 4), "fwd_tflops": round(ftf, 1),
                     "fwd_bwd_ms": round(ms, 4), "fwd_bwd_tflops": round(tf, 1),
                     "fwd_bwd_frac_fp32_peak": round(tf / FP32_PEAK_TFLOPS, 3)})
        log(f"  {case.name}: fwd {fwd_ms:.3f} ms ({ftf:.1f} TFLOP/s), fwd+bwd {ms:.3f} ms ({tf:.1f} TFLOP/s, "
            f"{tf / FP32_PEAK_TFLOPS:.0%} of the fp32 matrix peak)")
        del q, k, v, do
    return {"shape": "fp32 B4 H8, head_dim 64/128", "peak_tflops": FP32_PEAK_TFLOPS, "rows": rows}


def decode_suite(calls):
    """The pages' decode suite: one query per sequence, 32 query heads, head_dim 128, 8 or 32 KV heads.

    Full caches (no length mask). Each call's caches rotate over enough copies
    (>= 768 MiB in total) that they do not stay in the chip's last-level cache.
    """
    import math
    import torch
    from forward_backward_amd import attn
    from forward_backward_amd.inputs import workload_cases
    from forward_backward_amd.metrics import decode_bytes

    rows = []
    for case in workload_cases(6):
        kv_bytes = 2 * case.B * case.Tkv * case.Hkv * case.D * 2
        sets = max(1, min(16, math.ceil((768 << 20) / kv_bytes)))
        q = device_normal((case.B, case.Tq, case.Hq, case.D), 1)
        caches = [(device_normal((case.B, case.Tkv, case.Hkv, case.D), 2 + 2 * i),
                   device_normal((case.B, case.Tkv, case.Hkv, case.D), 3 + 2 * i)) for i in range(sets)]
        ws = attn.decode_workspace(q, caches[0][0])
        for i in range(2):
            attn.decode(q, *caches[i % sets], scale=case.scale, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        rounds = []
        for _ in range(3):  # median of three rounds, as the pages report
            e0.record()
            for i in range(calls):
                attn.decode(q, *caches[i % sets], scale=case.scale, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            rounds.append(e0.elapsed_time(e1) / calls * 1e3)
        us = sorted(rounds)[1]
        del ws
        mem = decode_memory(q, caches[0], None, case.scale)
        nbytes = decode_bytes(case.B, case.Tq, case.Hq, case.Hkv, case.D, [case.Tkv] * case.B)
        row = {"B": case.B, "keys": case.Tkv, "Hkv": case.Hkv, "us_per_call": round(us, 2),
               "us_rounds": [round(r, 2) for r in rounds],
               "gbs": round(nbytes / (us * 1e-6) / 1e9, 1), "bytes_per_call": nbytes, "cache_copies": sets,
               "workspace_bytes": mem["workspace_bytes"], "output_bytes": mem["output_bytes"],
               "device_peak_bytes": mem["device_peak_bytes"]}
        rows.append(row)
        log(f"  decode B{case.B} keys {case.Tkv} Hkv{case.Hkv}: {us:.1f} us/call, {row['gbs']} GB/s, workspace "
            f"{row['workspace_bytes'] / 2**20:.2f} MiB, peak {row['device_peak_bytes'] / 2**20:.2f} MiB")
        del q, caches
    return {"shape": "bf16 Tq=1 Hq32 d128, full caches, eager calls, median of three rounds",
            "memory": "workspace_bytes: attn_decode_workspace_size; output_bytes: O and LSE; device_peak_bytes: "
                      "one call that allocates its outputs and workspace, beyond the resident inputs",
            "rows": rows}


def cpu_baseline(case, seconds):
    """The float64 oracle on a bounded sample: whole (batch, KV head) groups of the headline workload."""
    import numpy as np
    from forward_backward_amd import inputs as I
    from forward_backward_amd.metrics import attention_flops
    import oracle

    host = I.make_inputs(case, seed=0)
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = len(os.sched_getaffinity(0))
    groups = [(b, kh) for b in range(case.B) for kh in range(case.Hkv)]
    done, t_used = 0, 0.0
    for b, kh in groups:
        sl = lambda x: I.to_float64(x[b:b + 1, :, kh:kh + 1], case.dtype)  # noqa: E731
        q, k, v, do = sl(host["q"]), sl(host["k"]), sl(host["v"]), sl(host["do"])
        t0 = time.perf_counter()
        oracle.attention_fwd(q, k, v, case.scale, case.causal)
        oracle.attention_bwd(q, k, v, do, case.scale, case.causal)
        t_used += time.perf_counter() - t0
        done += 1
        if t_used >= seconds:
            break
    flops = attention_flops(1, done, case.Tq, case.Tkv, case.D, case.causal, "fwd_bwd")
    return {
        "value": flops / t_used / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {len(groups)} (batch, head) groups of B4 H8 d128 T8192 non-causal, fwd then bwd, "
                  f"float64 NumPy, {t_used:.1f} s",
        "seconds": t_used,
    }


def blas_info():
    """The BLAS library NumPy runs on, and its thread count."""
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                return f"{p.get('internal_api')} {p.get('version')} ({os.path.basename(p.get('filepath', ''))})", \
                    int(p.get("num_threads", 1))
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass
    return "unknown", len(os.sched_getaffinity(0))


def cpu_oracle_configs():
    """The float64 oracle on every workload, forward and forward+backward timed separately, median of
    three calls; the two small workloads also with one thread. Large workloads are timed on a sample
    (one query head for the forward, one KV head with its query heads for the backward) and priced by
    the FLOPs of that sample; the KV-length workload samples one KV head per batch (the lengths
    differ), priced by the keys inside each length; decode runs whole. Sizes are chosen so that the
    whole table takes well under a minute on 16 host threads."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from forward_backward_amd import inputs as I
    from forward_backward_amd.inputs import workload_cases
    from forward_backward_amd.metrics import attention_flops, effective_flops
    import oracle

    blas, threads = blas_info()

    def med3(fn, reps=3):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[len(ts) // 2]

    def sample_slices(case, host, groups):
        out = []
        G = case.Hq // case.Hkv
        for b, kh in groups:
            sl = lambda x, hs: I.to_float64(x[b:b + 1, :, hs], case.dtype)  # noqa: E731
            lens = None if host["kv_lens"] is None else host["kv_lens"][b:b + 1]
            out.append(dict(q1=sl(host["q"], slice(kh * G, kh * G + 1)), qg=sl(host["q"], slice(kh * G, (kh + 1) * G)),
                            k=sl(host["k"], slice(kh, kh + 1)), v=sl(host["v"], slice(kh, kh + 1)),
                            do=sl(host["do"], slice(kh * G, (kh + 1) * G)), lens=lens, G=G))
        return out

    def time_case(case, groups, single=False, reps=3):
        host = I.make_inputs(case, seed=0)
        sm = sample_slices(case, host, groups)

        def fwd():
            for x in sm:
                oracle.attention_fwd(x["q1"], x["k"], x["v"], case.scale, case.causal, x["lens"], window=case.window)

        def fwd_bwd():
            for x in sm:
                oracle.attention_fwd(x["qg"], x["k"], x["v"], case.scale, case.causal, x["lens"], window=case.window)
                oracle.attention_bwd(x["qg"], x["k"], x["v"], x["do"], case.scale, case.causal, x["lens"],
                                     window=case.window)

        if case.kv_lens is not None or case.kv_len_range is not None:
            lens = [int(host["kv_lens"][b]) for b, _ in groups]
            f1 = effective_flops(1, case.Tq, lens, case.D, "fwd")
            fg = effective_flops(sm[0]["G"], case.Tq, lens, case.D, "fwd_bwd")
        else:
            f1 = len(groups) * attention_flops(1, 1, case.Tq, case.Tkv, case.D, case.causal, "fwd")
            fg = len(groups) * attention_flops(1, sm[0]["G"], case.Tq, case.Tkv, case.D, case.causal, "fwd_bwd")
        # fwd+bwd first: it also warms the allocation of the score-sized arrays the forward then reuses.
        fb = round(med3(fwd_bwd, reps) * 1e3, 3)
        row = {"workload": case.name, "sample": f"{len(groups)} of {case.B * case.Hkv} (batch, KV head) groups",
               "calls": reps, "fwd_ms": round(med3(fwd, reps) * 1e3, 3), "fwd_bwd_ms": fb}
        row["fwd_gflops"] = round(f1 / (row["fwd_ms"] * 1e-3) / 1e9, 2)
        row["fwd_bwd_gflops"] = round(fg / (row["fwd_bwd_ms"] * 1e-3) / 1e9, 2)
        if single:
            with threadpool_limits(limits=1, user_api="blas"):
                row["fwd_ms_1thread"] = round(med3(fwd) * 1e3, 3)
                row["fwd_bwd_ms_1thread"] = round(med3(fwd_bwd) * 1e3, 3)
        return row

    t_start = time.perf_counter()
    rows = []
    (c1,) = workload_cases(0)
    rows.append(time_case(c1, [(0, h) for h in range(c1.Hkv)], single=True))
    rows[-1]["sample"] = "whole workload"
    for case in workload_cases(1):
        rows.append(time_case(case, [(0, 0)], single=case.Tq <= 1024))
    for case in workload_cases(2):
        rows.append(time_case(case, [(0, 0)], reps=1))
    (c4,) = workload_cases(3)
    rows.append(time_case(c4, [(b, 0) for b in range(c4.B)], reps=1))
    (c5,) = workload_cases(4)
    host = I.make_inputs(c5, seed=0, with_do=False)
    f64 = {n: I.to_float64(host[n], c5.dtype) for n in ("q", "k", "v")}
    dec_ms = med3(lambda: oracle.attention_decode(f64["q"], f64["k"], f64["v"], c5.scale, host["kv_lens"])) * 1e3
    fl = effective_flops(c5.Hq, c5.Tq, host["kv_lens"], c5.D, "fwd")
    rows.append({"workload": c5.name, "sample": "whole workload", "calls": 3, "fwd_ms": round(dec_ms, 3),
                 "fwd_gflops": round(fl / (dec_ms * 1e-3) / 1e9, 2)})
    log(f"  oracle per workload: {time.perf_counter() - t_start:.1f} s")
    return {"blas": blas, "threads": threads,
            "unit": "ms per call of the sample (median of `calls`); GFLOP/s of the sample", "rows": rows}


STALL_COUNTERS = {
    "SQ_WAVE_CYCLES": "wave-cycles (quad-cycles) the kernel's waves were resident",
    "SQ_ACTIVE_INST_ANY": "wave-cycles an instruction of the wave was being executed",
    "SQ_WAIT_ANY": "wave-cycles spent waiting on anything (s_waitcnt, barrier, dependency)",
    "SQ_WAIT_INST_ANY": "wave-cycles spent waiting for an issue slot",
    "SQ_WAIT_INST_LDS": "wave-cycles spent waiting to issue an LDS instruction",
    "SQ_ACTIVE_INST_VALU": "wave-cycles on VALU instructions",
    "SQ_ACTIVE_INST_LDS": "wave-cycles on LDS instructions",
    "SQ_VALU_MFMA_BUSY_CYCLES": "cycles the matrix units were busy (all SIMDs)",
    "SQ_VALU_MFMA_COEXEC_CYCLES": "of those, cycles in which a VALU instruction was issued too",
    "SQ_INSTS_MFMA": "MFMA instructions",
    "SQ_INSTS_VALU": "VALU instructions",
    "SQ_INSTS_SALU": "SALU instructions",
    "SQ_INSTS_LDS": "LDS instructions",
    "SQ_LDS_BANK_CONFLICT": "LDS bank-conflict cycles",
    "SQ_LDS_IDX_ACTIVE": "LDS busy cycles",
}


def summarize_stalls(pmc_dirs, command, out_dir=""):
    """Per-kernel issue and wait counters of the headline run, and the ratios read from them."""
    import csv
    import glob
    names = {}
    for d in pmc_dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                names.setdefault(r["Counter_Name"], d)
    per = {}
    for c, d in names.items():
        if c not in STALL_COUNTERS:
            continue
        for (k, grid), vals in _read_counter_csv(d, c).items():
            if k.startswith("attn"):
                per.setdefault((k, grid), {})[c] = sum(vals) / len(vals)
    lines = ["# Issue and wait counters: attention fwd+bwd B4 H8 d128 T8192, non-causal", "",
             "rocprofv3 counter passes (one per line of the command block; each pass stays within the per-block "
             "counter limits) over the same run. Values are per dispatch, averaged over the dispatches of a "
             "kernel and grid. The ratio columns: `co-issue` = SQ_VALU_MFMA_COEXEC_CYCLES / "
             "SQ_VALU_MFMA_BUSY_CYCLES (share of matrix-busy cycles in which a VALU instruction issued too); "
             "`wait`, `issue wait` and `active` = SQ_WAIT_ANY, SQ_WAIT_INST_ANY and SQ_ACTIVE_INST_ANY over "
             "SQ_WAVE_CYCLES; `VALU/MFMA`, `SALU/MFMA` and `LDS/MFMA` = instruction counts per MFMA.", "",
             "```", command or "", "```", "",
             "| kernel | grid | co-issue | wait | issue wait | active | VALU/MFMA | SALU/MFMA | LDS/MFMA | "
             "LDS bank conflicts |", "|---|---|---|---|---|---|---|---|---|---|"]

    def ratio(cs, a, b, pct=True):
        if a not in cs or b not in cs or cs[b] == 0:
            return "-"
        v = cs[a] / cs[b]
        return f"{100 * v:.0f}%" if pct else f"{v:.2f}"

    for (k, grid), cs in sorted(per.items()):
        if not cs.get("SQ_INSTS_MFMA"):
            continue
        lines.append(f"| `{k}` | {grid} | {ratio(cs, 'SQ_VALU_MFMA_COEXEC_CYCLES', 'SQ_VALU_MFMA_BUSY_CYCLES')} | "
                     f"{ratio(cs, 'SQ_WAIT_ANY', 'SQ_WAVE_CYCLES')} | {ratio(cs, 'SQ_WAIT_INST_ANY', 'SQ_WAVE_CYCLES')} | "
                     f"{ratio(cs, 'SQ_ACTIVE_INST_ANY', 'SQ_WAVE_CYCLES')} | "
                     f"{ratio(cs, 'SQ_INSTS_VALU', 'SQ_INSTS_MFMA', False)} | "
                     f"{ratio(cs, 'SQ_INSTS_SALU', 'SQ_INSTS_MFMA', False)} | "
                     f"{ratio(cs, 'SQ_INSTS_LDS', 'SQ_INSTS_MFMA', False)} | {cs.get('SQ_LDS_BANK_CONFLICT', 0):.0f} |")
    lines += ["", "Raw values (per dispatch):", "", "| kernel | counter | value | meaning |", "|---|---|---|---|"]
    for (k, grid), cs in sorted(per.items()):
        for c in sorted(cs):
            lines.append(f"| `{k}` | {c} | {cs[c]:.4g} | {STALL_COUNTERS[c]} |")
    prof = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    path = os.path.join(prof, "fwd_bwd_d128_T8192_issue_counters.md")
    open(path, "w").write("\n".join(lines) + "\n")
    log(f"wrote {path}")


def summarize_suites(log_path, command, out_dir=""):
    """Markdown tables of every leg and suite of one bench line."""
    line = [x for x in open(log_path) if x.startswith("{")][-1]
    d = json.loads(line)
    L = ["# Every leg of one bench run: headline, causal, window, decode, short sequences, KV lengths, suites",
         "", "One `bench.py` run on one MI355X (the JSON line it printed, in tables). Command:", "",
         "```", command or "(not recorded)", "```", ""]
    sp = d.get("timing_spread", {}).get("per_step_ms", {})
    L += ["## Headline (bf16 B4 H8 d128 T8192, non-causal, fwd+bwd)", "",
          f"- {d['value']} TFLOP/s over {d['steps']} timed steps ({d['ms_per_step']} ms per step, mean); "
          f"per step median {sp.get('median')} ms, quartiles {sp.get('q1')} / {sp.get('q3')} ms",
          f"- per kernel ms (mean): {d['per_kernel_ms']}",
          f"- roofline of `{d['roofline']['kernel']}`: {d['roofline']['achieved']} TFLOP/s, "
          f"{d['roofline']['frac']:.1%} of {d['roofline']['peak']}", ""]
    if "causal" in d:
        c = d["causal"]
        L += [f"- causal: {c['ms_per_step']} ms, {c['tflops']} TFLOP/s; per kernel {c['per_kernel_ms']}"]
    if "window" in d:
        w = d["window"]
        L += [f"- causal 1024-key window: {w['ms_per_step']} ms, {w['tflops_visible']} TFLOP/s over visible pairs"]
    if "decode" in d:
        x = d["decode"]
        r = x["roofline"]
        L += [f"- GQA decode (B4, 32 query heads over 8 KV heads, 16 queries, 16384-key caches, lengths "
              f"{x['kv_lens']}): {x['us_per_call']} us per call in a graph ({r['achieved']} GB/s algorithmic, "
              f"{r['frac']:.1%} of HBM; counter traffic {r.get('traffic')} B); eager {x['us_per_call_eager']} us; "
              f"memory {x.get('memory')}"]
    L.append("")
    if "short_sequences" in d:
        L += ["## Short sequences (bf16 B4 H8 d64)", "", "| case | fwd us | fwd TFLOP/s | fwd+bwd us | fwd+bwd TFLOP/s |",
              "|---|---|---|---|---|"]
        L += [f"| {r['case']} | {r['fwd_us']} | {r['fwd_tflops']} | {r['fwd_bwd_us']} | {r['fwd_bwd_tflops']} |"
              for r in d["short_sequences"]["rows"]]
        L.append("")
    if "kv_len" in d:
        x = d["kv_len"]
        L += [f"KV-length workload ({x['workload']}, lengths {x['kv_lens']}): fwd+bwd {x['fwd_bwd_ms']} ms, "
              f"{x['effective_tflops']} TFLOP/s over the keys inside the lengths ({x['nominal_tflops']} nominal).", ""]
    if "gqa_suite" in d:
        L += ["## GQA suite (bf16 B1, 32 query heads over 8 KV heads, d128, fwd+bwd)", "",
              "| T | ms | TFLOP/s | peak MB | repeated K/V ms | repeated K/V peak MB |", "|---|---|---|---|---|---|"]
        L += [f"| {r['T']} | {r['ms']} | {r['tflops']} | {r['peak_mb']} | {r['repeated_ms']} | {r['repeated_peak_mb']} |"
              for r in d["gqa_suite"]["rows"]]
        L.append("")
    if "decode_suite" in d:
        L += ["## Decode suite (bf16, one query, 32 query heads, d128, full caches; median of three rounds)", "",
              "| B | keys | KV heads | us per call | GB/s | workspace MiB | output bytes | device peak MiB |",
              "|---|---|---|---|---|---|---|---|"]
        L += [f"| {r['B']} | {r['keys']} | {r['Hkv']} | {r['us_per_call']} | {r['gbs']} | "
              f"{r['workspace_bytes'] / 2**20:.2f} | {r['output_bytes']} | {r['device_peak_bytes'] / 2**20:.2f} |"
              for r in d["decode_suite"]["rows"]]
        L.append("")
    if "headdim_sweep" in d:
        L += ["## head_dim sweep (bf16 B4 H8 T4096, fwd+bwd)", "", "| D | ms | TFLOP/s |", "|---|---|---|"]
        L += [f"| {r['D']} | {r['ms']} | {r['tflops']} |" for r in d["headdim_sweep"]["rows"]]
        L.append("")
    if "config_grid" in d:
        L += ["## head_dim-64 grid (bf16 B4 H8)", "", "| case | fwd ms | fwd TFLOP/s | fwd+bwd ms | fwd+bwd TFLOP/s |",
              "|---|---|---|---|---|"]
        L += [f"| {r['case']} | {r['fwd_ms']} | {r['fwd_tflops']} | {r['fwd_bwd_ms']} | {r['fwd_bwd_tflops']} |"
              for r in d["config_grid"]["head_dim64_grid"]["rows"]]
        L.append("")
    if "memory" in d:
        m = d["memory"]
        L += ["## Memory", "", "| fwd+bwd bf16 B4 H8 d64, T | device peak MB beyond inputs | inputs MB |", "|---|---|---|"]
        L += [f"| {r['T']} | {r['device_peak_mb']} | {r['inputs_mb']} |" for r in m["device_peak"]["rows"]]
        L += ["", "| bytes kept for the backward, bf16 B2 H8 d64, T | MB (O and LSE) |", "|---|---|"]
        L += [f"| {r['T']} | {r['residual_mb']} |" for r in m["residuals"]["rows"]]
        L.append("")
    if "fp32_suite" in d:
        L += ["## fp32 grid (B4 H8)", "", "| case | fwd ms | fwd TFLOP/s | fwd+bwd ms | fwd+bwd TFLOP/s | of fp32 peak |",
              "|---|---|---|---|---|---|"]
        L += [f"| {r['case']} | {r['fwd_ms']} | {r['fwd_tflops']} | {r['fwd_bwd_ms']} | {r['fwd_bwd_tflops']} | "
              f"{r['fwd_bwd_frac_fp32_peak']:.0%} |" for r in d["fp32_suite"]["rows"]]
        L.append("")
    if d.get("cpu_baseline"):
        c = d["cpu_baseline"]
        L += ["## CPU oracle (float64 NumPy on the host cores)", "",
              f"Headline sample: {c['value'] * 1e3:.1f} GFLOP/s on {c['cores']} threads ({c['sample']}); BLAS "
              f"{c.get('blas')}.", ""]
        pw = c.get("per_workload")
        if pw:
            L += [f"Per workload ({pw['unit']}; {pw['threads']} BLAS threads):", "",
                  "| workload | sample | calls | fwd ms | fwd+bwd ms | fwd ms, 1 thread | fwd+bwd ms, 1 thread |",
                  "|---|---|---|---|---|---|---|"]
            L += [f"| {r['workload']} | {r['sample']} | {r.get('calls', 3)} | {r.get('fwd_ms')} | {r.get('fwd_bwd_ms', '-')} | "
                  f"{r.get('fwd_ms_1thread', '-')} | {r.get('fwd_bwd_ms_1thread', '-')} |" for r in pw["rows"]]
            L.append("")
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), "suites_and_legs.md")
    with open(path, "w") as f:
        f.write("\n".join(L) + "\n")
    print(f"wrote {path}")


def main():
    args = parse_args()
    if args.summarize_suites:
        summarize_suites(args.summarize_suites, args.profile_command)
        return
    if args.summarize_stalls:
        summarize_stalls(args.summarize_stalls, args.counter_command)
        return
    if args.summarize_fp32:
        summarize_fp32(args.summarize_fp32, args.profile_command)
        return
    if args.summarize:
        summarize(*args.summarize, args.profile_command, args.counter_command)
        if args.mfma_dir:
            summarize_mfma(args.summarize[0], args.mfma_dir, args.mfma_command, args.profile_command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from forward_backward_amd import attn
    from forward_backward_amd.inputs import workload_cases
    from forward_backward_amd.metrics import PEAK_HBM_GBS, PEAK_TFLOPS, attention_flops, decode_bytes, visible_pairs

    attn.lib()  # fail loudly without the HIP library
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')} CUs {props.multi_processor_count}")

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes")
        del src, dst

    full, causal = workload_cases(2)
    log(f"headline {full.name}: warmup {args.warmup}, steps {args.steps}")
    ms, per, dist = time_train_steps(full, args.steps, args.warmup, spread=True)
    flops = attention_flops(full.B, full.Hq, full.Tq, full.Tkv, full.D, False, "fwd_bwd")
    tflops = flops / (ms * 1e-3) / 1e12
    step_q = dist["step_ms"]
    spread = {"per_step_ms": step_q,
              "tflops_at": {k: round(flops / (step_q[v] * 1e-3) / 1e12, 2) for k, v in
                            (("median", "median"), ("q1_time", "q1"), ("q3_time", "q3"))},
              "per_kernel_ms": dist["per_kernel_ms"],
              "note": "median and quartiles over the K timed steps (HIP events around each step and kernel)"}
    log(f"  {ms:.3f} ms/step, {tflops:.1f} TFLOP/s; per kernel ms: " +
        ", ".join(f"{k} {v:.3f}" for k, v in per.items()))

    fwd_f = attention_flops(full.B, full.Hq, full.Tq, full.Tkv, full.D, False, "fwd")
    kernel_flops = {"attn_fwd": fwd_f, "bwd_dkdv": 2 * fwd_f, "bwd_dq": 1.5 * fwd_f}
    kernel_symbol = KERNEL_SYMBOLS
    dom = max(kernel_flops, key=lambda n: per[n])
    achieved = kernel_flops[dom] / (per[dom] * 1e-3) / 1e12
    roofline = {
        "bound": "mfma",
        "kernel": kernel_symbol[dom],
        "achieved": round(achieved, 2),
        "peak": PEAK_TFLOPS["bf16"],
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
        "traffic": stored_traffic(kernel_symbol[dom]),
        "avg_ms": round(per[dom], 4),
        "flops_per_launch": kernel_flops[dom],
    }

    extra = {"timing_spread": spread}
    if not args.no_extra:
        log(f"causal {causal.name}")
        cms, cper = time_train_steps(causal, args.steps, 1)
        cfl = attention_flops(causal.B, causal.Hq, causal.Tq, causal.Tkv, causal.D, True, "fwd_bwd")
        extra["causal"] = {"ms_per_step": round(cms, 4), "tflops": round(cfl / (cms * 1e-3) / 1e12, 2),
                           "per_kernel_ms": {k: round(v, 4) for k, v in cper.items()}}
        log(f"  {cms:.3f} ms/step, {extra['causal']['tflops']} TFLOP/s")
        (win,) = workload_cases(7)
        log(f"window {win.name}")
        wms, wper = time_train_steps(win, args.steps, 1)
        pairs = visible_pairs(win.Tq, win.Tkv, win.causal, win.window)
        wfl = 3.5 * 4.0 * win.B * win.Hq * win.D * pairs
        extra["window"] = {"workload": win.name, "ms_per_step": round(wms, 4),
                           "tflops_visible": round(wfl / (wms * 1e-3) / 1e12, 2),
                           "visible_pairs_per_head": pairs,
                           "flop_count": "3.5 * 4 * B * H * D * visible (query, key) pairs",
                           "per_kernel_ms": {k: round(v, 4) for k, v in wper.items()}}
        log(f"  {wms:.3f} ms/step, {extra['window']['tflops_visible']} TFLOP/s over visible pairs")
        (dec,) = workload_cases(4)
        graph_ms, cold, warm, lens, dmem = time_decode(dec, args.decode_calls)
        nbytes = decode_bytes(dec.B, dec.Tq, dec.Hq, dec.Hkv, dec.D, lens)
        gbs = nbytes / (graph_ms * 1e-3) / 1e9
        counted = [stored_traffic(KERNEL_SYMBOLS[k]) for k in ("decode_split", "decode_combine")]
        counter_bytes = sum(counted) if all(c is not None for c in counted) else None
        extra["decode"] = {
            "workload": dec.name, "kv_lens": lens, "us_per_call": round(graph_ms * 1e3, 2),
            "timing": "HIP graph of captured calls, 4 K/V caches in rotation",
            "us_per_call_eager": round(cold * 1e3, 2), "us_per_call_same_cache_eager": round(warm * 1e3, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_call": nbytes,
                         "traffic": counter_bytes,
                         "counter_gbs": None if counter_bytes is None else
                         round(counter_bytes / (graph_ms * 1e-3) / 1e9, 1),
                         "traffic_note": "FETCH_SIZE + WRITE_SIZE of the split and combine kernels per call, "
                                         "scaled by a plain copy (profiles/hbm_traffic.json); null when the "
                                         "kernel sources changed since the counters were taken"},
            "memory": dmem,
        }
        log(f"decode {graph_ms * 1e3:.1f} us/call in a graph ({gbs:.0f} GB/s); eager {cold * 1e3:.1f} us, "
            f"same cache {warm * 1e3:.1f} us")
        log("short sequences and the KV-length workload")
        extra["short_sequences"], extra["kv_len"] = short_and_kvlen_legs(max(args.steps, 20))

    if args.gemm_ceiling:
        log("bf16 GEMM through torch (hipBLASLt)")
        extra["gemm_ceiling"] = gemm_ceiling()
    if args.suites:
        log("GQA suite")
        extra["gqa_suite"] = gqa_suite(max(2, min(args.steps, 5)))
        log("decode suite")
        extra["decode_suite"] = decode_suite(50)
        log("head_dim sweep")
        extra["headdim_sweep"] = headdim_sweep(max(2, min(args.steps, 5)))
        log("head_dim 64 grid and KV-length case")
        extra["config_grid"] = config_grid(max(2, min(args.steps, 5)))
        log("memory")
        extra["memory"] = memory_suite()
    if args.suites or args.fp32_suite:
        log("fp32 suite")
        extra["fp32_suite"] = fp32_suite(max(2, min(args.steps, 5)))

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (float64 oracle)")
        cpu = cpu_baseline(full, args.cpu_seconds)
        log(f"  {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads ({cpu['sample']})")
        cpu["blas"] = blas_info()[0]
        cpu["per_workload"] = cpu_oracle_configs()

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: i.i.d. N(0,1) bf16 from seed 0",
        "config": {"workload": "bf16 MHA fwd+bwd B4 H8 d128 Tq=Tkv=8192 non-causal", "B": 4, "H": 8, "D": 128,
                   "T": 8192, "causal": False},
        "mfma_peak_frac": round(tflops / PEAK_TFLOPS["bf16"], 4),
        "per_kernel_ms": {k: round(v, 4) for k, v in per.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        **extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
