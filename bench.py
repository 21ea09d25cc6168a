#!/usr/bin/env python3
"""Throughput of the sparse MoE layer hot path on one MI355X.

One step = one moe_forward call (router GEMM, softmax/top-k, permute,
grouped gate|up+SwiGLU and down FFN, combine) over one batch of seeded
synthetic input already resident in HBM.  W untimed warm-up steps, then
exactly K timed steps bracketed by torch.cuda.synchronize(); before each
step an untimed 1 GiB fill evicts the L2 caches and the 256 MiB MALL, and a
HIP event pair on the launch stream times the step itself.  `value` is the
token count over the median step time; the minimum and mean are reported
beside it.  Prints one JSON line.  The routed expert weights are re-laid out
once (moe_pack_weights) before anything is timed, as a serving engine does at
load time, and the plain layout is then freed: only the packed copy stays
resident.  --no-packed keeps the plain layout instead.

Default workload: one decode step of a Qwen-3.5-like layer (T=64 tokens,
H=4096, E=512 experts, top-10, I=1024, bf16 experts, fp32 router).

Also reported:
  roofline      the dominant kernel launch (largest duration; a kernel run twice
                per step, as the heavy GEMMs with a shared expert, is timed per
                launch), timed with HIP events on its own launch stream over
                the timed region, against
                the HBM (or bf16 MFMA) peak; traffic from committed rocprofv3
                counter summaries when they match the current kernel source.
  cpu_baseline  the CPU oracle timed on this host on a bounded sample.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FLUSH_BYTES = 1 << 30          # untimed fill before each timed step (> L2 + 256 MiB MALL)
NEAR_TIE = 1e-6                # k-th vs (k+1)-th probability gap flagged as a near-tie
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", default="decode",
                   help="workload: decode (default), prefill, prefill_long, skew, ling, tiny")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=64, help="tokens in the oracle's sample")
    p.add_argument("--no-packed", action="store_true",
                   help="the light loop reads the plain weight layout instead of the packed "
                        "copy made once before timing (moe_pack_weights)")
    p.add_argument("--y-dtype", choices=("auto", "fp32", "bf16", "fp16"), default="auto",
                   help="storage of the routed expert outputs between the down GEMM and the "
                        "combine; auto = bf16, fp16 for a layer with a shared expert (its "
                        "outputs need more than bf16's 8 bits), fp32 for fp32-valued layers")
    p.add_argument("--weights", choices=("bf16", "mxfp8"), default="bf16",
                   help="routed expert weights: bf16, or MXFP8 (OCP MX E4M3 codes with one "
                        "E8M0 scale per 32 values, quantised on the GPU before timing)")
    p.add_argument("--heavy-tile-rows", type=int, default=0, choices=(0, 128, 160, 192, 224, 256),
                   help="heavy tile height: 0 = the library's per-expert choice (results do "
                        "not depend on it)")
    p.add_argument("--no-copy-calibration", action="store_true",
                   help="skip the untimed 1 GiB reference copy used to scale rocprof counters")
    p.add_argument("--summarize", nargs=4, metavar=("KT_DIR", "FETCH_DIR", "WRITE_DIR", "LOG"),
                   help="no GPU: turn the rocprofv3 output of the three profiling runs of "
                        "--config (and the kernel-trace run's stdout LOG) into the summaries "
                        "under profiles/")
    p.add_argument("--summarize-mfma", nargs=3, metavar=("KT_DIR", "PMC_DIR", "LOG"),
                   help="no GPU: MFMA pipe occupancy and clock of the heavy GEMMs from a "
                        "kernel-trace run and a SQ_VALU_MFMA_BUSY_CYCLES + GRBM_GUI_ACTIVE run "
                        "of --config -> profiles/mfma_busy__<workload>.md")
    return p.parse_args()


# The runs that profiles/mfma_busy__<workload>.md summarises ($R as below).
MFMA_COMMANDS = (
    "rocprofv3 --kernel-trace --stats -f csv -d $R/gpurun_out/mkt_{cfg}{tag} -o bench -- "
    "python3 $R/bench.py --config {cfg}{extra} --steps 5 --warmup 1 --no-cpu-baseline "
    "> $R/gpurun_out/mkt_{cfg}{tag}.log",
    "timeout -s KILL 150 rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE -f csv "
    "-d $R/gpurun_out/mfma_{cfg}{tag} -o bench -- python3 $R/bench.py --config {cfg}{extra} "
    "--steps 3 --warmup 1 --no-cpu-baseline",
    "python3 $R/bench.py --config {cfg}{extra} --summarize-mfma $R/gpurun_out/mkt_{cfg}{tag} "
    "$R/gpurun_out/mfma_{cfg}{tag} $R/gpurun_out/mkt_{cfg}{tag}.log",
)
N_CU, SIMD_PER_CU, N_XCD = 256, 4, 8


def summarize_mfma(args):
    """MFMA pipe occupancy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x
    CUs x 4 SIMDs) per launch, averaged over a kernel's launches; the clock
    the chip held = GRBM_GUI_ACTIVE / the kernel-trace average duration."""
    import csv
    import collections
    from expert_ffn_layer_amd import synth

    kt_dir, pmc_dir, log = args.summarize_mfma
    cfg = synth.CONFIGS[args.config]
    workload = workload_of(cfg, args.weights)

    def one_csv(d, suffix):
        names = [f for f in os.listdir(d) if f.endswith(suffix)]
        assert len(names) == 1, (d, names)
        with open(os.path.join(d, names[0])) as f:
            return list(csv.DictReader(f))

    dur = collections.defaultdict(list)
    for r in one_csv(kt_dir, "kernel_stats.csv"):
        lab = kernel_label(r["Name"])
        if lab in ("gateup_heavy", "down_heavy", "gateup_light", "down_light", "router_gemm"):
            dur[lab].append((float(r["TotalDurationNs"]), int(r["Calls"])))
    # Per dispatch: the MFMA busy cycles summed over the chip, and
    # GRBM_GUI_ACTIVE, which rocprofv3 reports as one value summed over the
    # 8 XCDs (each XCD counts the cycles the GPU is busy): /8 gives the cycles.
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    span = {}
    for r in one_csv(pmc_dir, "counter_collection.csv"):
        lab = kernel_label(r["Kernel_Name"])
        if lab in dur:
            key = (lab, r["Dispatch_Id"])
            per[key][r["Counter_Name"]] += float(r["Counter_Value"])
            span[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    rows = {}
    for lab in dur:
        ks = [k for k in per if k[0] == lab and per[k].get("GRBM_GUI_ACTIVE")]
        tot_ns = sum(t for t, _ in dur[lab])
        calls = sum(c for _, c in dur[lab])
        avg_us = tot_ns / calls / 1e3
        if not ks or avg_us < 50:  # empty or tiny launches: counts dominated by launch overhead
            continue
        cyc = [per[k]["GRBM_GUI_ACTIVE"] / N_XCD for k in ks]
        busy = sum(per[k]["SQ_VALU_MFMA_BUSY_CYCLES"] / (c * N_CU * SIMD_PER_CU)
                   for k, c in zip(ks, cyc)) / len(ks)
        mhz = sum(c / span[k] for k, c in zip(ks, cyc)) / len(ks) / 1e6
        rows[lab] = (busy, avg_us, mhz, len(ks))
    with open(log) as f:
        line = [l for l in f if l.startswith("{")][-1]
    rec = json.loads(line)
    rf = rec["roofline"]
    tag = "" if args.weights == "bf16" else f"_{args.weights}"
    extra = "" if args.weights == "bf16" else f" --weights {args.weights}"
    cmds = [c.format(cfg=args.config, tag=tag, extra=extra) for c in MFMA_COMMANDS]
    lines = [f"# MFMA pipe occupancy on {workload}", "",
             "rocprofv3 counters of bench.py on one MI355X (gfx950).  Commands, from /tmp with",
             "TMPDIR=/tmp, $R the repository root:", "", "```", *cmds, "```", "",
             f"Occupancy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x {N_CU} CUs x "
             f"{SIMD_PER_CU} SIMDs), per launch, averaged, with GRBM_GUI_ACTIVE (reported summed "
             f"over the {N_XCD} XCDs) divided by {N_XCD}; clock = those cycles over the "
             "launch's own start-to-end time in the counter run.  Kernels of 50 us and more.", "",
             "| kernel | launches counted | avg us | MFMA pipes busy | clock MHz |",
             "|---|---|---|---|---|"]
    for lab, (busy, avg_us, mhz, n) in sorted(rows.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"| {lab} | {n} | {avg_us:.1f} | {100 * busy:.1f}% | {mhz:.0f} |")
    lines += ["", f"bench line: {rec['value']:.1f} tokens/s, {rec['ms_per_step']:.4f} ms/step; "
                  f"{rf['kernel']} at {rf['flops'] / (rf['kernel_us'] * 1e-6) / 1e12:.1f} TFLOP/s "
                  f"of expert FLOPs = {100 * rf['flops'] / (rf['kernel_us'] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS:.1f}% "
                  f"of the {BF16_PEAK_TFLOPS:.0f} TFLOP/s bf16 dense peak."]
    path = os.path.join(PROFILES, f"mfma_busy__{workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {path}")


# The profiling runs that profiles/<kernel>__<workload>.{md,traffic.json}
# summarise; $R is the repository root, run from /tmp with TMPDIR=/tmp.
PROFILE_COMMANDS = (
    "rocprofv3 --kernel-trace --stats -f csv -d $R/gpurun_out/kt_{cfg}{tag} -o bench -- "
    "python3 $R/bench.py --config {cfg}{extra} --steps 10 --warmup 2 --no-cpu-baseline "
    "> $R/gpurun_out/kt_{cfg}{tag}.log",
    "timeout -s KILL 150 rocprofv3 --pmc FETCH_SIZE -f csv -d $R/gpurun_out/fetch_{cfg}{tag} -o bench -- "
    "python3 $R/bench.py --config {cfg}{extra} --steps 3 --warmup 1 --no-cpu-baseline",
    "timeout -s KILL 150 rocprofv3 --pmc WRITE_SIZE -f csv -d $R/gpurun_out/write_{cfg}{tag} -o bench -- "
    "python3 $R/bench.py --config {cfg}{extra} --steps 3 --warmup 1 --no-cpu-baseline",
    "python3 $R/bench.py --config {cfg}{extra} --summarize $R/gpurun_out/kt_{cfg}{tag} "
    "$R/gpurun_out/fetch_{cfg}{tag} $R/gpurun_out/write_{cfg}{tag} $R/gpurun_out/kt_{cfg}{tag}.log",
)


def composite_lower_bound(router_bytes, router_flops, ffn_bytes, ffn_flops) -> float:
    """Seconds a layer needs at the least when the router and then the FFN
    each run at the roofline that binds them: max(router bytes / HBM peak,
    router FLOPs / fp32 peak) + max(FFN bytes / HBM peak, FFN FLOPs / bf16
    peak)."""
    bw = HBM_PEAK_GBS * 1e9
    return (max(router_bytes / bw, router_flops / (FP32_PEAK_TFLOPS * 1e12)) +
            max(ffn_bytes / bw, ffn_flops / (BF16_PEAK_TFLOPS * 1e12)))


def workload_of(cfg, weights: str) -> str:
    """Workload name: the layer's shape, plus the weight format when not bf16."""
    from expert_ffn_layer_amd import synth
    return synth.workload_name(cfg) + ("" if weights == "bf16" else f"_{weights}")
# bench.py's own untimed reference copy (torch.neg over 2^28 fp32 values):
# it reads and writes exactly 1 GiB.
COPY_BYTES = 1 << 30


def kernel_label(name: str):
    """The KERNELS name of a rocprof kernel name, or None if it is not ours."""
    import re
    m = re.search(r"moe::\(anonymous namespace\)::(\w+)", name)
    if not m:
        return None
    base = m.group(1)
    if base.endswith("_mx_kernel"):  # MXFP8-weight variants of the light loops
        base = base[:-len("_mx_kernel")] + "_kernel"
    if base == "ffn_heavy_kernel":
        return "gateup_heavy" if "Mode)0" in name else "down_heavy"
    if base.startswith("router_select"):  # block- and wave-per-token variants
        return "router_select"
    return base[:-len("_kernel")] if base.endswith("_kernel") else base


def summarize(args):
    """Per-kernel duration (kernel trace) and HBM traffic (FETCH_SIZE and
    WRITE_SIZE in KiB per dispatch, each scaled by what the counter reads for
    the 1 GiB reference copy) -> profiles/<dominant>__<workload>.md and
    .traffic.json."""
    import csv
    from expert_ffn_layer_amd import synth

    kt_dir, fetch_dir, write_dir, log = args.summarize
    cfg = synth.CONFIGS[args.config]
    workload = workload_of(cfg, args.weights)

    def one_csv(d, suffix):
        names = [f for f in os.listdir(d) if f.endswith(suffix)]
        assert len(names) == 1, (d, names)
        with open(os.path.join(d, names[0])) as f:
            return list(csv.DictReader(f))

    # A kernel's instances (template arguments) are different launches: the
    # heavy GEMMs of a layer with a shared expert run one instance for the
    # routed experts and another for the shared one.  The table sums them per
    # step; the dominant kernel's own line and traffic take its largest
    # instance, the launch bench.py times (the routed one).
    stats, inst = {}, {}
    for r in one_csv(kt_dir, "kernel_stats.csv"):
        lab = kernel_label(r["Name"])
        if not lab:
            continue
        cur = dict(calls=int(r["Calls"]), min_us=float(r["MinNs"]) / 1e3,
                   max_us=float(r["MaxNs"]) / 1e3, total_us=float(r["TotalDurationNs"]) / 1e3)
        inst[r["Name"]] = dict(cur, label=lab, avg_us=cur["total_us"] / cur["calls"])
        if lab in stats:
            prev = stats[lab]
            big = prev if prev["total_us"] >= cur["total_us"] else cur
            cur = dict(calls=max(prev["calls"], cur["calls"]), min_us=big["min_us"],
                       max_us=big["max_us"], total_us=prev["total_us"] + cur["total_us"])
        stats[lab] = cur
    for st_ in stats.values():
        st_["avg_us"] = st_["total_us"] / st_["calls"]

    def counter(d):
        per, copy = {}, None
        for r in one_csv(d, "counter_collection.csv"):
            v = float(r["Counter_Value"])
            if "neg_kernel_cuda" in r["Kernel_Name"]:
                copy = v
                continue
            lab = kernel_label(r["Kernel_Name"])
            if lab:
                per.setdefault(lab, {}).setdefault(r["Kernel_Name"], []).append(v)
        assert copy, f"no reference copy kernel in {d}"
        scale = COPY_BYTES / (copy * 1024.0)
        by_label = {k: sum(sum(v) / len(v) for v in ins.values()) * 1024.0 * scale
                    for k, ins in per.items()}
        by_inst = {n: sum(v) / len(v) * 1024.0 * scale
                   for ins in per.values() for n, v in ins.items()}
        return by_label, by_inst, scale

    fetch, fetch_i, f_scale = counter(fetch_dir)
    write, write_i, w_scale = counter(write_dir)
    rec = None
    with open(log) as f:
        for line in f:
            if line.startswith('{"metric"'):
                rec = json.loads(line)
    assert rec and rec["config"]["workload"] == workload, "log is not this workload's bench line"
    dom = max(stats, key=lambda k: stats[k]["total_us"])
    src_hash = rec["kernel_source_hash"]
    assert src_hash == kernel_source_hash(), "kernel sources changed since the profiled run"

    dom_inst = max((n for n in inst if inst[n]["label"] == dom), key=lambda n: inst[n]["total_us"])
    n_inst = sum(1 for n in inst if inst[n]["label"] == dom)
    d_avg, d_calls = inst[dom_inst]["avg_us"], inst[dom_inst]["calls"]
    f_dom = fetch_i.get(dom_inst, fetch[dom])
    w_dom = write_i.get(dom_inst, write[dom])
    traffic = f_dom + w_dom
    roof = rec["roofline"]
    out = {"kernel": dom, "workload": workload, "kernel_source_hash": src_hash,
           "hbm_bytes_per_launch": int(round(traffic)),
           "fetch_bytes_per_launch": int(round(f_dom)),
           "write_bytes_per_launch": int(round(w_dom)),
           "fetch_size_scale": round(f_scale, 4), "write_size_scale": round(w_scale, 4),
           "algorithmic_bytes_per_launch": roof["algorithmic_bytes"] if roof["kernel"] == dom
           else None,
           "avg_duration_us": round(d_avg, 2)}
    base = os.path.join(PROFILES, f"{dom}__{workload}")
    os.makedirs(PROFILES, exist_ok=True)
    with open(base + ".traffic.json", "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")

    mxw = args.weights != "bf16"
    cmds = "\n".join(c.format(cfg=args.config, tag=f"_{args.weights}" if mxw else "",
                              extra=f" --weights {args.weights}" if mxw else "")
                     for c in PROFILE_COMMANDS)
    lines = [f"# {dom} on {workload}", "",
             "rocprofv3 summary of bench.py on one MI355X (gfx950).  Commands, from /tmp with",
             "TMPDIR=/tmp, $R the repository root:", "", "```", cmds, "```", "",
             f"Dominant kernel: **{dom}**, average {d_avg:.1f} us over "
             f"{d_calls} calls (kernel trace"
             + (f"; its largest of {n_inst} instances, the launch timed below; the table sums "
                f"the instances per step" if n_inst > 1 else "")
             + f"); bench.py's own HIP-event timing of it in the same run: "
             f"{roof['kernel_us']:.1f} us.",
             "", f"bench line: {rec['value']:.1f} {rec['unit']}, {rec['ms_per_step']:.4f} ms/step; "
             f"roofline {roof['bound']} {roof['achieved']} {roof['unit']} "
             f"(frac {roof['frac']}) for {roof['kernel']}.", "",
             f"Counter scale: FETCH_SIZE x {f_scale:.4f}, WRITE_SIZE x {w_scale:.4f} (the "
             "counters' readings for bench.py's untimed 1 GiB read + 1 GiB write reference "
             "copy).", "",
             "| kernel | calls | avg us | min us | max us | HBM read MB/launch | "
             "HBM write MB/launch |", "|---|---|---|---|---|---|---|"]
    for k in sorted(stats, key=lambda k: -stats[k]["total_us"]):
        st = stats[k]
        lines.append(f"| {k} | {st['calls']} | {st['avg_us']:.1f} | {st['min_us']:.1f} | "
                     f"{st['max_us']:.1f} | {fetch.get(k, 0) / 1e6:.2f} | "
                     f"{write.get(k, 0) / 1e6:.2f} |")
    alg = out["algorithmic_bytes_per_launch"]
    if alg:
        lines += ["", f"{dom}: measured HBM traffic {traffic / 1e6:.1f} MB per launch against "
                      f"{alg / 1e6:.1f} MB algorithmic ({traffic / alg:.2f}x)."]
    with open(base + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {base}.md and .traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "expert_ffn_layer_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from profiles/<kernel>__<workload>.traffic.json,
    or None when absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, f"{kernel}__{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.summarize:
        summarize(args)
        return
    if args.summarize_mfma:
        summarize_mfma(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from expert_ffn_layer_amd import moe, synth

    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload {synth.workload_name(cfg)}: generating", file=sys.stderr, flush=True)
    layer = synth.make_layer(cfg, seed=args.seed, device=dev)
    if cfg.fp32_values:
        layer = layer.rounded_to_bf16()
    y_dt = args.y_dtype
    if y_dt == "auto":
        y_dt = "fp32" if cfg.fp32_values else ("fp16" if cfg.I_shared else "bf16")
    mx = args.weights == "mxfp8"
    m = moe.MoELayer(layer, packed=not args.no_packed, y_bf16=y_dt == "bf16",
                     weights=args.weights, y_fp16=y_dt == "fp16",
                     heavy_tile_rows=args.heavy_tile_rows)
    s = m.shape
    # The oracle's inputs for the CPU baseline (its sample's tokens and the
    # experts they reach) are copied to the host before the plain weights
    # are freed; then only the packed copy of the expert weights is resident.
    cpu_in = None if args.no_cpu_baseline else cpu_baseline_inputs(layer, cfg, args.cpu_sample)
    if m.packed is not None:
        layer.w_gu = layer.w_dn = None
        torch.cuda.empty_cache()
    w_gu_arg, w_dn_arg = layer.w_gu, layer.w_dn
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=dev)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    counts = torch.empty((cfg.E,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        moe.forward(s, layer.x, layer.wg, layer.bias, w_gu_arg, w_dn_arg, layer.ws_gu,
                    layer.ws_dn, out, m.workspace, ids, w, counts, stream=stream,
                    packed_weights=m.packed)

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()

    # Untimed pass: per-kernel durations, to name the dominant launch.  A
    # kernel launched more than once per step (the heavy GEMMs of a layer with
    # a shared expert: routed experts, then the shared one) is timed launch by
    # launch; its per-step time is the sum.
    per_kernel, per_launch = {}, {}
    for name in moe.KERNELS:
        a0, b0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        moe.profile_kernel(name, a0, b0)
        step()
        n_launch = moe.profile_launches()
        moe.profile_kernel(None)
        torch.cuda.synchronize()
        if n_launch == 0:  # kernels this workload does not launch are left out
            continue
        for i in range(n_launch):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(2)]
            for a, b in ev:
                moe.profile_kernel(name, a, b, launch=i)
                step()
            moe.profile_kernel(None)
            torch.cuda.synchronize()
            per_launch[(name, i)] = sum(a.elapsed_time(b) for a, b in ev) / len(ev) * 1e3  # us
        per_kernel[name] = sum(v for (k, _), v in per_launch.items() if k == name)
    dominant, dom_launch = max(per_launch, key=per_launch.get)

    # Timed region: K steps, each after an untimed 1 GiB fill that evicts the
    # caches, timed by its own event pair on the launch stream; the dominant
    # kernel's launch is bracketed by events each step too.
    # The fill leaves its lines dirty in L2 and MALL; reading a second buffer
    # of the same size afterwards writes them back and leaves clean lines, so
    # no write-back of the fill lands inside the timed step.
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_rd = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)
    mk = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    evs = [mk() for _ in range(args.steps)]
    step_evs = [mk() for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps (dominant kernel {dominant})", file=sys.stderr,
          flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, ((a, b), (sa, sb)) in enumerate(zip(evs, step_evs)):
        flush.fill_(float(i))
        torch.sum(flush_rd, dim=0, out=flush_sink)
        sa.record(stream)
        moe.profile_kernel(dominant, a, b, launch=dom_launch)
        step()
        sb.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    moe.profile_kernel(None)
    del flush, flush_rd
    step_ms = sorted(sa.elapsed_time(sb) for sa, sb in step_evs)
    ms_per_step = float(np.median(step_ms))
    wall_ms_per_step = (t1 - t0) * 1e3 / args.steps
    kern_us = sum(a.elapsed_time(b) for a, b in evs) / len(evs) * 1e3
    value = cfg.T / (ms_per_step / 1e3)

    # Algorithmic work, from this run's own routing.
    cnt = counts.cpu().numpy().astype(np.int64)
    touched = int((cnt > 0).sum())
    routing = routing_stats(s, layer, cnt, cfg, m.workspace)
    light = moe.light_experts(cnt, s)
    light_rows = int(cnt[light].sum())
    light_experts = int(light.sum())
    A = cfg.T * cfg.k
    H, I = cfg.H, cfg.I
    x_bytes = cfg.T * H * 2
    y_el = 4 if y_dt == "fp32" else 2  # bytes per stored y value
    Is = cfg.I_shared
    # Bytes of one routed expert's weights as the kernels stream them: bf16,
    # or MXFP8 codes (W_down's K padded to 64) plus a scale byte per 32.
    if mx:
        i_pad = (I + 63) // 64 * 64
        gu_w = 2 * I * H * (1 + 1 / 32)
        dn_w = H * i_pad * (1 + 1 / 32)
    else:
        gu_w, dn_w = 2 * I * H * 2, H * I * 2
    if dominant == "gateup_heavy" and dom_launch == 1:  # the shared expert, dense over T
        alg = 2 * Is * H * 2 + x_bytes + cfg.T * 2 * Is * 2  # h kept as a bf16 hi|lo pair
        flops = 4 * cfg.T * H * Is
    elif dominant == "down_heavy" and dom_launch == 1:
        alg = H * Is * 2 + cfg.T * 2 * Is * 2 + cfg.T * H * 4
        flops = 2 * cfg.T * H * Is
    elif dominant == "gateup_light":
        alg = light_experts * gu_w + x_bytes + light_rows * I * 2
        flops = 4 * light_rows * H * I
    elif dominant == "down_light":
        alg = light_experts * dn_w + light_rows * (I * 2 + H * y_el)
        flops = 2 * light_rows * H * I
    elif dominant == "gateup_heavy":
        he = touched - light_experts
        hr = A - light_rows
        alg = he * gu_w + x_bytes + hr * I * 2
        flops = 4 * hr * H * I
    elif dominant == "down_heavy":
        he = touched - light_experts
        hr = A - light_rows
        alg = he * dn_w + hr * (I * 2 + H * y_el)
        flops = 2 * hr * H * I
    elif dominant == "router_gemm":
        alg = x_bytes + H * cfg.E * 4
        flops = 2 * cfg.T * H * cfg.E
    elif dominant == "combine":
        alg = A * H * y_el + cfg.T * H * 4 * (2 if Is else 1)  # out also read when accumulating
        flops = 0
    else:
        alg, flops = 0, 0
    t_k = kern_us * 1e-6
    t_hbm = alg / (HBM_PEAK_GBS * 1e9)
    peak_flops = FP32_PEAK_TFLOPS if dominant == "router_gemm" else BF16_PEAK_TFLOPS
    t_mfma = flops / (peak_flops * 1e12)
    src_hash = kernel_source_hash()
    workload = workload_of(cfg, args.weights)
    # (committed counter summaries cover a kernel's first launch of a step)
    traffic = committed_traffic(dominant, workload, src_hash) if dom_launch == 0 else None
    if t_mfma > t_hbm:
        achieved = flops / t_k / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_flops,
                "unit": "TFLOP/s", "frac": round(achieved / peak_flops, 4)}
    else:
        achieved = alg / t_k / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": traffic, "kernel": dominant, "launch": dom_launch,
                 "kernel_us": round(kern_us, 2),
                 "algorithmic_bytes": int(alg), "flops": int(flops)})

    # Whole-layer roofline (weights of touched experts + x + router + out).
    layer_bytes = int(touched * (gu_w + dn_w)) + x_bytes + H * cfg.E * 4 + cfg.T * H * 4
    if cfg.I_shared:
        layer_bytes += 3 * H * cfg.I_shared * 2
    layer_flops = 6 * A * H * I + (6 * cfg.T * H * cfg.I_shared if cfg.I_shared else 0)
    t_step = ms_per_step / 1e3
    # Composite bound: the router (x and W_g read; its FLOPs at the fp32
    # peak, the precision it is defined in) followed by the FFN (touched and
    # shared expert weights, out written; expert FLOPs at the bf16 peak),
    # each at whichever of its two rooflines binds.
    t_lb = composite_lower_bound(x_bytes + H * cfg.E * 4, 2 * cfg.T * H * cfg.E,
                                 layer_bytes - x_bytes - H * cfg.E * 4, layer_flops)
    layer = dict(hbm_frac=round(layer_bytes / t_step / (HBM_PEAK_GBS * 1e9), 4),
                 mfma_frac=round(layer_flops / t_step / (BF16_PEAK_TFLOPS * 1e12), 4),
                 composite_frac=round(t_lb / t_step, 4), composite_lb_us=round(t_lb * 1e6, 2),
                 algorithmic_bytes=int(layer_bytes), expert_flops=int(layer_flops),
                 touched_experts=touched, light_experts=light_experts)

    # Untimed reference copy: 1 GiB read + 1 GiB written by one elementwise
    # kernel, the yardstick for rocprof FETCH_SIZE / WRITE_SIZE.
    if not args.no_copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if cpu_in is not None:
        cpu = cpu_baseline(cpu_in, cfg=cfg, gpu_out=out, mx=mx)

    rec = {
        "metric": "MoE-layer tokens/s",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms": {"median": round(ms_per_step, 4), "min": round(step_ms[0], 4),
                    "mean": round(float(np.mean(step_ms)), 4),
                    "wall_incl_flush": round(wall_ms_per_step, 4),
                    "timing": "HIP events around each moe_forward, after an untimed "
                              f"{FLUSH_BYTES >> 20} MiB fill that evicts L2 and MALL and "
                              f"an untimed {FLUSH_BYTES >> 20} MiB read of another buffer "
                              "that writes the fill's dirty lines back"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the MFMAs multiply bf16 operands (MXFP8 codes are converted to bf16
        # operands exactly, before the MFMA)
        "dtype": "mxfp8-weights/bf16" if mx else "bf16",
        "data": "synthetic (seeded normal draws, random-init weights)",
        "config": {"workload": workload, "tokens": cfg.T, "hidden": H, "experts": cfg.E,
                   "top_k": cfg.k, "intermediate": I, "shared_intermediate": cfg.I_shared,
                   "seed": args.seed, "packed_weights": m.packed is not None,
                   "y_dtype": y_dt,
                   "weights": "mxfp8 (E4M3, E8M0 per 32)" if mx else "bf16"},
        "roofline": roof,
        "layer_roofline": layer,
        "routing": routing,
        "kernels_us": {k: round(v, 2) for k, v in per_kernel.items()},
        "kernel_source_hash": src_hash,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def routing_stats(shape, layer_obj, cnt, cfg, ws):
    """The routing this step saw: rows per expert (max, min, experts with at
    most 3 rows, the top 10% of experts' share of all rows) and near-ties
    (tokens whose k-th and (k+1)-th softmax probabilities, as the GPU router
    computes them, are within 1e-6; and tokens with two adjacent ranks among
    the first k+1 that close).  One untimed moe_router call with probs."""
    import numpy as np
    import torch

    from expert_ffn_layer_amd import moe

    A = cfg.T * cfg.k
    srt = np.sort(cnt)[::-1]
    top = max(1, cfg.E // 10)
    st = {"max_rows": int(cnt.max()), "min_rows": int(cnt.min()),
          "experts_le3_rows": int((cnt <= 3).sum()), "touched_experts": int((cnt > 0).sum()),
          "top10pct_share": round(float(srt[:top].sum()) / A, 4)}
    dev = layer_obj.x.device
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    probs = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev)
    moe.router(shape, layer_obj.x, layer_obj.wg, layer_obj.bias, ids, w, probs, ws)
    kk = min(cfg.k + 1, cfg.E)
    p = torch.topk(probs, kk, dim=1).values.cpu().numpy().astype(np.float64)
    gaps = p[:, :-1] - p[:, 1:]
    set_doubt = (gaps[:, cfg.k - 1] < NEAR_TIE) if kk > cfg.k else np.zeros(cfg.T, bool)
    order_doubt = (gaps < NEAR_TIE).any(axis=1) & ~set_doubt
    st["near_ties"] = {"kth_vs_next": int(set_doubt.sum()), "order_within_topk": int(order_doubt.sum()),
                       "threshold": NEAR_TIE, "from": "GPU router probabilities"}
    del probs
    return st


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline_inputs(layer_obj, cfg, n):
    """Host copies of what the oracle reads for the first n tokens: their
    activations, the router, the shared expert, and the routed experts the
    oracle's own routing of those tokens reaches (untimed)."""
    import numpy as np

    import oracle

    n = min(n, cfg.T)
    o = oracle.Oracle()
    x = layer_obj.x[:n].cpu()
    wg = layer_obj.wg.cpu()
    bias = None if layer_obj.bias is None else layer_obj.bias.cpu()
    r = o.route(o.logits(x, wg, bias), cfg.k, cfg.renorm)
    experts = [int(e) for e in np.unique(r["ids"])]
    print(f"[bench] cpu baseline: copying {len(experts)} experts to host", file=sys.stderr,
          flush=True)
    return dict(n=n, x=x, wg=wg, bias=bias,
                w_gu={e: layer_obj.w_gu[e].cpu() for e in experts},
                w_dn={e: layer_obj.w_dn[e].cpu() for e in experts},
                ws_gu=None if layer_obj.ws_gu is None else layer_obj.ws_gu.cpu(),
                ws_dn=None if layer_obj.ws_dn is None else layer_obj.ws_dn.cpu())


def cpu_baseline(inp, cfg, gpu_out, mx=False):
    """The oracle (plain fp32 C loops, OpenMP over rows) on the first n tokens
    of the same layer, weights already on the host; also reports its
    agreement with the GPU output on those tokens.  With MXFP8 weights the
    oracle first quantises and dequantises (untimed) the experts those tokens
    reach, then runs the same forward on them."""
    import numpy as np
    import torch

    import oracle

    n = inp["n"]
    o = oracle.Oracle()
    w_gu, w_dn = inp["w_gu"], inp["w_dn"]
    if mx:
        deq_gu, deq_dn = {}, {}
        for e in w_gu:
            for src, dst in ((w_gu, deq_gu), (w_dn, deq_dn)):
                c, sc = o.mxfp8_quantize(src[e].float().numpy())
                dst[e] = o.mxfp8_dequantize(c, sc)
        w_gu, w_dn = deq_gu, deq_dn
    print(f"[bench] cpu baseline: oracle on {n} tokens", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    ref = o.forward(inp["x"], inp["wg"], inp["bias"], w_gu, w_dn, cfg.k, cfg.renorm,
                    inp["ws_gu"], inp["ws_dn"], permute=False)
    wall = time.perf_counter() - t0
    g = gpu_out[:n].cpu().numpy().astype(np.float64)
    d = g - ref["out"].astype(np.float64)
    torch.cuda.synchronize()
    return {"value": round(n / wall, 3), "unit": "tokens/s", "cores": o.max_threads(),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "kind": "oracle",
            "sample": f"first {n} of {cfg.T} tokens of the same layer (routing, all their expert "
                      f"FFN rows, combine); fp32 C loops; expert weights pre-copied to host"
                      + (" (MXFP8-dequantised by the oracle, untimed)" if mx else ""),
            "wall_s": round(wall, 3),
            "gpu_vs_oracle": {"max_abs": float(np.abs(d).max()),
                              "rel_l2": float(np.linalg.norm(d) / np.linalg.norm(ref["out"]))}}


if __name__ == "__main__":
    main()
