"""Benchmark of the Nystrom self-attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--config NAME|all]
                    [--no-cpu-baseline] [--cpu-1thread]

Workload: B=16, H=8, n=4096, d=64, m=64 landmarks (segments of 64 tokens), depthwise
conv width 33, 6 pseudo-inverse iterations, bf16 I/O; seeded synthetic Q, K, V ~ N(0,1)
and conv weights (stand-ins for the GLUE/IMDB/LRA inputs of the pages, which are not
available). A step is one full forward (segment means, landmark kernel and iterative
pseudo-inverse, landmark context, output softmax times Y, conv skip) with inputs already
resident in HBM; consecutive steps alternate between two independently seeded input
sets so no step starts with its inputs cache-resident.

Untimed forwards for a fixed second come first (the GPU's clock ramp), then W warm-up
steps, then exactly K timed steps. Prints one JSON line per workload: tokens/s (tokens =
B*n per forward), the whole forward against its binding roofline term (HBM, MFMA or VALU,
from algorithmic counts), per-kernel times from HIP events recorded by the library on the
forward's stream (and from the committed rocprofv3 summary when it matches the sources),
and the fp64 CPU oracle timed on the host on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Nyström attn fwd tokens/s at n=4096,m=64,d=64; % of binding roofline"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "efficient_transformer_attention_segment_amd", "csrc")
STAGES = ("segment_means", "pinv", "context", "output")
# kernel name (as rocprofv3 reports it) of each stage; for m <= 64 the pseudo-inverse
# blocks run inside context_kernel and the "pinv" stage is empty
STAGE_KERNEL = {"segment_means": "segmeans_kernel", "pinv": "pinv_global_kernel",
                "context": "context_kernel", "output": "output_kernel"}


def stage_bytes(cfg, lengths=None) -> dict:
    """Algorithmic HBM bytes per launch of each stage (inputs read once, output written
    once; the small landmark-sized workspace traffic is not counted). With padded
    lengths only valid rows are read; every output row is written (zeros on padding)."""
    e = 2 if cfg.dtype == "bf16" else 4
    valid = cfg.n * cfg.B if lengths is None else sum(lengths)
    tok = cfg.H * valid * cfg.d * e
    full = cfg.bh * cfg.n * cfg.d * e
    return {"segment_means": 2 * tok,      # read Q, K
            "pinv": 0,                     # landmark-sized only (compute/latency bound)
            "context": 2 * tok,            # read K, V
            "output": 2 * tok + full}      # read Q, V; write out


# MI355X peaks (AMD's published figures): HBM3E, dense MFMA, vector fp32, and the
# transcendental rate assumed for v_exp_f32 (a quarter of the fp32 lane rate: 16 lanes
# per clock per CU at 2.4 GHz on 256 CUs).
PEAK_HBM = 8.0e12          # B/s
PEAK_MFMA_BF16 = 2.5e15    # flop/s
PEAK_MFMA_F32 = 157.3e12   # flop/s
PEAK_VALU_F32 = 157.3e12   # flop/s
PEAK_EXP = 256 * 16 * 2.4e9


def path_roofline(cfg, lengths=None) -> dict:
    """The forward's roofline from algorithmic counts: t_roof = max(T_HBM, T_MFMA,
    T_VALU) with
      T_HBM  = (Q, K, V read once + out written once) / 8 TB/s;
      T_MFMA = 8 n m d per head (the two scores and the two probability products) at the
               dense bf16 rate (fp32 rate for fp32 I/O), plus the landmark work per head,
               8 T m^3 (T iterations of four m x m products) + 4 m^2 d (A_S logits,
               Y = Z W), counted as three bf16 products per product since the
               pseudo-inverse runs on hi/lo bf16 pairs;
      T_VALU = 2 W n d per head (the conv skip) at the fp32 vector rate + the (2 n m + m^2)
               exponentials per head at the v_exp rate.
    Only valid tokens count for a padded batch. Dense O(n^2) work is never counted."""
    e = 2 if cfg.dtype == "bf16" else 4
    tokens = cfg.n * cfg.B if lengths is None else sum(lengths)
    th = cfg.H * tokens                      # token-heads processed
    n_m_d = th * cfg.m * cfg.d
    hbm = 3 * th * cfg.d * e + cfg.bh * cfg.n * cfg.d * e
    land = cfg.bh * (8 * cfg.pinv_iters * cfg.m ** 3 + 4 * cfg.m ** 2 * cfg.d)
    if cfg.dtype == "bf16":
        t_mfma = 8 * n_m_d / PEAK_MFMA_BF16 + 3 * land / PEAK_MFMA_BF16
    else:
        t_mfma = 8 * n_m_d / PEAK_MFMA_F32 + land / PEAK_MFMA_F32
    flops_mfma = 8 * n_m_d + land
    t_valu = 2 * cfg.conv_width * th * cfg.d / PEAK_VALU_F32 + \
        (2 * th * cfg.m + cfg.bh * cfg.m ** 2) / PEAK_EXP
    terms = {"hbm": hbm / PEAK_HBM, "mfma": t_mfma, "valu": t_valu}
    bound = max(terms, key=terms.get)
    return {"bound": bound, "t_roof_s": terms[bound], "terms_s": terms,
            "algorithmic_bytes": hbm, "mfma_flops": flops_mfma}


def roofline_record(cfg, ms: float, lengths=None) -> dict:
    """The forward as one unit against its binding roofline term: achieved = that term's
    algorithmic work / measured time, frac = t_roof / t."""
    pr = path_roofline(cfg, lengths)
    t = ms * 1e-3
    if pr["bound"] == "hbm":
        achieved, peak, unit = pr["algorithmic_bytes"] / t / 1e9, PEAK_HBM / 1e9, "GB/s"
    elif pr["bound"] == "mfma":
        peak = (PEAK_MFMA_BF16 if cfg.dtype == "bf16" else PEAK_MFMA_F32) / 1e12
        achieved, unit = pr["t_roof_s"] * peak / t, "TFLOP/s (bf16-equivalent)"
    else:
        achieved, peak, unit = pr["t_roof_s"] * PEAK_VALU_F32 / 1e12 / t, PEAK_VALU_F32 / 1e12, \
            "TFLOP/s (fp32-equivalent)"
    return {"kernel": "whole forward (all stages)", "bound": pr["bound"],
            "achieved": achieved, "peak": peak, "unit": unit, "frac": pr["t_roof_s"] / t,
            "t_roof_ms": pr["t_roof_s"] * 1e3,
            "terms_ms": {k: v * 1e3 for k, v in pr["terms_s"].items()},
            "algorithmic_bytes": pr["algorithmic_bytes"], "mfma_flops": pr["mfma_flops"]}


def source_hash(stage: str) -> str:
    files = {"segment_means": ["segmeans.hip"], "pinv": ["context.hip"],
             "context": ["context.hip"], "output": ["output.hip"]}[stage]
    files += ["nys_common.h", "nys_kernels.h", "plan.hip"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(stage: str, cfg_name: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None when the
    kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{STAGE_KERNEL[stage]}_{cfg_name}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != source_hash(stage):
        return None
    return rec.get("traffic_bytes_per_launch")


def traced_kernel_us(cfg_name: str) -> dict:
    """Kernel time of each stage per forward (us) from the committed rocprofv3
    kernel-trace summary of this workload, when it was taken on the current sources."""
    path = os.path.join(PROFILES, f"nystrom_forward_{cfg_name}_kernel_trace.txt")
    if not os.path.exists(path):
        return {}
    with open(path) as fh:
        text = fh.read()
    if "sources " + "/".join(source_hash(s) for s in STAGES) not in text:
        return {}
    out = {}
    for line in text.splitlines():
        parts = line.split()
        if len(parts) == 3 and parts[0] == "stage_us":
            out[parts[1]] = float(parts[2])
    return out


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(cfg, x, budget_s: float = 12.0, lengths=None, threads=None) -> dict:
    """Time the fp64 oracle (untuned) on the host on a bounded sample of the workload:
    its heads in order, one at a time, until about budget_s seconds have passed (whole
    passes over all heads while the budget allows). tokens/s counts the tokens of the
    sampled heads divided by H, i.e. B n tokens per full pass. threads: BLAS threads
    (default: as configured)."""
    import contextlib
    import oracle
    ctx = contextlib.nullcontext()
    if threads is not None:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=threads)
    lens = [cfg.n] * cfg.B if lengths is None else list(lengths)
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    with ctx:
        cores = _blas_threads()
        done, tok = 0, 0
        t0 = time.perf_counter()
        while True:
            b, h = heads[done % len(heads)]
            oracle.nystrom_forward(x.q, x.k, x.v, x.w, cfg.m, cfg.pinv_iters, heads=[(b, h)],
                                   lengths=lengths)
            done += 1
            tok += lens[b]
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    return {"value": tok / cfg.H / dt, "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} head forward(s) of the workload's {cfg.bh} heads "
                      f"({done / cfg.bh:.2f} full passes) in {dt:.1f} s, numpy fp64, "
                      f"BLAS threads={cores}"}


# ------------------------------------------------------------------ profile summaries
# rocprofv3 output -> short text summaries under profiles/ (no GPU needed)

def _short(name: str) -> str:
    name = name.replace("void ", "")
    return name.split("(")[0].replace("nys::", "")


KERNEL_STAGE = (("segmeans", "segment_means"), ("pinv", "pinv"), ("context", "context"),
                ("output", "output"))


def summarize_trace(trace_dir: str, cfg_name: str, command: str,
                    title: str = "the Nystrom attention forward") -> str:
    """Per-kernel dispatch count and mean duration from a rocprofv3 --kernel-trace
    --stats database: over all dispatches (what --stats reports) and over the last 200
    (the event-profiled forwards that bench.py's stage times come from); then the kernel
    time of each forward stage per forward over the last 200 forwards (one forward = one
    output-kernel dispatch), tagged with the hash of the sources it was taken on."""
    import glob
    import sqlite3
    db = sorted(glob.glob(os.path.join(trace_dir, "**", "*.db"), recursive=True))[0]
    con = sqlite3.connect(db)
    rows = con.execute("select name, total_calls, average from top_kernels").fetchall()
    seq = con.execute("select name, duration from kernels order by start").fetchall()
    per = {}
    for name, dur in seq:
        per.setdefault(name, []).append(dur)
    lines = [f"Kernel trace of {title}, workload {cfg_name} "
             f"({CONFIG_TEXT.get(cfg_name, cfg_name)}), one MI355X.", "",
             "Command (repository root; rocprofv3 wants the program right after --):",
             f"  {command}", "",
             f"{'kernel':64s} {'calls':>6s} {'avg_us':>9s} {'last200_us':>11s}"]
    for name, calls, avg in rows:
        d = per.get(name, [])
        tail = sum(d[-200:]) / max(1, len(d[-200:])) / 1e3
        lines.append(f"{_short(name)[:64]:64s} {calls:6d} {avg:9.3f} {tail:11.3f}")
    outs = [i for i, (name, _) in enumerate(seq) if _short(name).startswith("output_kernel")]
    if len(outs) > 200 and title == "the Nystrom attention forward":
        first = outs[-201] + 1
        stage_us = {st: 0.0 for _, st in KERNEL_STAGE}
        for name, dur in seq[first:outs[-1] + 1]:
            for prefix, st in KERNEL_STAGE:
                if _short(name).startswith(prefix):
                    stage_us[st] += dur / 1e3 / 200
        lines += ["", "Kernel time per forward over the last 200 forwards (us), sources "
                  + "/".join(source_hash(s) for s in STAGES) + ":"]
        lines += [f"stage_us {st} {stage_us[st]:.3f}" for _, st in KERNEL_STAGE]
    return "\n".join(lines) + "\n"


def _read_counters(d: str):
    import csv
    import glob
    out = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"],
                            float(r["Counter_Value"])))
    return out


def summarize_counters(fetch_dir: str, write_dir: str, cfg_name: str, commands) -> dict:
    """HBM traffic per launch of each kernel from a FETCH_SIZE run and a WRITE_SIZE run
    (KiB per dispatch), each scaled by what the counter reads for the 256 MiB device
    copies of --copy-calibration (known to read and write 256 MiB)."""
    fetch = _read_counters(fetch_dir)
    write = _read_counters(write_dir)
    cal_kib = 256 * 1024
    cal_ids = [i for i, n, c, v in write
               if "copyBuffer" in n and c == "WRITE_SIZE" and abs(v - cal_kib) < 0.1 * cal_kib]
    cw = [v for i, n, c, v in write if i in cal_ids and c == "WRITE_SIZE"]
    cf = [v for i, n, c, v in fetch if i in cal_ids and c == "FETCH_SIZE"]
    if not cw or not cf:
        raise SystemExit("no calibration copies found (run with --copy-calibration)")
    wscale, fscale = cal_kib / (sum(cw) / len(cw)), cal_kib / (sum(cf) / len(cf))
    res = {}
    for stage, kern in STAGE_KERNEL.items():
        fv = [v for i, n, c, v in fetch if _short(n).startswith(kern + "<") and c == "FETCH_SIZE"]
        wv = [v for i, n, c, v in write if _short(n).startswith(kern + "<") and c == "WRITE_SIZE"]
        if not fv or not wv:
            continue
        f_kib, w_kib = sum(fv) / len(fv), sum(wv) / len(wv)
        res[kern] = {
            "kernel": kern, "workload": cfg_name, "source_hash": source_hash(stage),
            "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
            "fetch_scale": fscale, "write_scale": wscale,
            "calibration": "256 MiB device copies (hipMemcpy D2D kernel): counter KiB "
                           "-> true KiB",
            "traffic_bytes_per_launch": (f_kib * fscale + w_kib * wscale) * 1024,
            "commands": list(commands)}
    return res


CONFIG_TEXT = {"long": "B=16 H=8 n=4096 d=64 m=64, conv width 33, 6 pseudo-inverse "
                       "iterations, bf16 I/O",
               "bert": "B=32 H=12 n=512 d=64 m=64, conv width 33, 6 pseudo-inverse "
                       "iterations, bf16 I/O",
               "large_m": "B=4 H=8 n=16384 d=64 m=256, conv width 33, 6 pseudo-inverse "
                          "iterations, bf16 I/O",
               "very_long": "B=2 H=16 n=65536 d=128 m=128, conv width 33, 6 pseudo-inverse "
                            "iterations, bf16 I/O, Q and K of variance 2"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--ramp-s", type=float, default=1.0,
                    help="untimed forwards for this many seconds before the warm-up "
                         "(reported as clock_ramp)")
    ap.add_argument("--config", default="long",
                    help="workload name, or 'all' for one JSON line per workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--cpu-1thread", action="store_true",
                    help="also time the oracle with one BLAS thread (cpu_baseline_1thread)")
    ap.add_argument("--ragged", action="store_true",
                    help="padded batch: seeded valid lengths in [n/2, n] per batch element "
                         "(tokens/s then counts valid tokens)")
    ap.add_argument("--layer", type=int, metavar="D", default=0,
                    help="time the projected layer instead: Q/K/V projection from model "
                         "width D, the forward, and the output projection back to D")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (gradients of sum(out * dout) for Q, K, V "
                         "and the conv weights) instead of the forward")
    ap.add_argument("--flash", type=int, metavar="CHUNK", default=0,
                    help="time FLASH mixed-chunk attention with this chunk size instead")
    ap.add_argument("--causal", action="store_true", help="with --flash: causal variant")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write profiles/nystrom_forward_<config>_kernel_trace.txt from a "
                         "rocprofv3 --kernel-trace --stats output directory and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/<kernel>_<config>_counters.json from rocprofv3 "
                         "--pmc FETCH_SIZE and --pmc WRITE_SIZE output directories and exit")
    ap.add_argument("--trace-name", default="nystrom_forward",
                    help="with --summarize-trace: file name stem of the summary")
    ap.add_argument("--trace-title", default="the Nystrom attention forward",
                    help="with --summarize-trace: what the trace covers")
    ap.add_argument("--command", action="append", default=[],
                    help="command line(s) that produced the summarized output")
    args = ap.parse_args()
    if args.summarize_trace:
        os.makedirs(PROFILES, exist_ok=True)
        path = os.path.join(PROFILES, f"{args.trace_name}_{args.config}_kernel_trace.txt")
        with open(path, "w") as fh:
            fh.write(summarize_trace(args.summarize_trace, args.config, " && ".join(args.command),
                                     args.trace_title))
        print(f"wrote {path}")
        return
    if args.summarize_counters:
        os.makedirs(PROFILES, exist_ok=True)
        for kern, rec in summarize_counters(*args.summarize_counters, args.config,
                                            args.command).items():
            path = os.path.join(PROFILES, f"{kern}_{args.config}_counters.json")
            with open(path, "w") as fh:
                json.dump(rec, fh, indent=1)
            print(f"wrote {path}")
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the forward shards over (batch, head) without communication; see the "
              "design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from efficient_transformer_attention_segment_amd import inputs as gen

    torch.cuda.set_device(0)
    names = gen.CONFIG_ORDER if args.config == "all" else [args.config]
    for name in names:
        cfg = gen.CONFIGS[name]
        if args.layer:
            layer_bench(args, cfg)
        elif args.backward:
            backward_bench(args, cfg)
        elif args.flash:
            flash_bench(args, cfg)
        else:
            forward_bench(args, name)
        torch.cuda.empty_cache()


def clock_ramp(step, seconds: float) -> dict:
    """Untimed forwards for a fixed wall time before the warm-up: the GPU leaves its idle
    clocks only after some milliseconds of work, so a short timed run would otherwise
    measure the ramp rather than the kernels."""
    import torch
    t0, done = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step(done)
            done += 1
        torch.cuda.synchronize()
    return {"seconds": round(time.perf_counter() - t0, 3), "forwards": done}


def forward_bench(args, name: str):
    """Steps of the Nystrom forward on one workload; one JSON line."""
    import torch
    from efficient_transformer_attention_segment_amd import NystromAttention
    from efficient_transformer_attention_segment_amd import inputs as gen
    cfg = gen.CONFIGS[name]
    sets = [gen.make_inputs(cfg), gen.make_inputs(cfg, seed=cfg.seed + 1000)]

    def dev(a):
        if cfg.dtype == gen.BF16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    dev_sets = [(dev(s.q_dev), dev(s.k_dev), dev(s.v_dev), torch.from_numpy(s.w).cuda())
                for s in sets]
    dt = torch.bfloat16 if cfg.dtype == gen.BF16 else torch.float32
    outs = [torch.empty(cfg.B, cfg.H, cfg.n, cfg.d, dtype=dt, device="cuda") for _ in sets]
    att = NystromAttention(cfg.B, cfg.H, cfg.n, cfg.d, cfg.m, cfg.conv_width,
                           cfg.pinv_iters, cfg.dtype)

    lengths = gen.ragged_lengths(cfg, cfg.seed) if args.ragged else None
    lens_dev = torch.tensor(lengths, dtype=torch.int32, device="cuda") if lengths else None

    def step(i):
        q, k, v, w = dev_sets[i % 2]
        att.forward(q, k, v, w, out=outs[i % 2], lengths=lens_dev)

    ramp = clock_ramp(step, args.ramp_s)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps

    # per-stage kernel times: HIP events the library records on the forward's stream
    # (each interval also holds the gap before its launch)
    nprof = min(max(args.steps, 20), 200)
    att.profile_enable(nprof)
    for i in range(nprof):
        step(i)
    torch.cuda.synchronize()
    prof = np.array(att.profile_read(nprof), dtype=np.float64)
    stage_ms = {s: float(prof[:, j].mean()) for j, s in enumerate(STAGES)}

    if args.copy_calibration:
        a = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()

    tokens = cfg.tokens if lengths is None else sum(lengths)
    value = tokens / (ms * 1e-3)
    sbytes = stage_bytes(cfg, lengths)
    roof = roofline_record(cfg, ms, lengths)
    traffic = None
    if lengths is None:
        parts = [measured_traffic(st, name) for st in ("segment_means", "context", "output")]
        traffic = sum(parts) if all(p is not None for p in parts) else None
    roof["traffic"] = traffic
    traced = {} if lengths else traced_kernel_us(name)
    kernels = {}
    for st in STAGES:
        rec_k = {"event_ms": stage_ms[st], "algorithmic_bytes": sbytes[st]}
        if sbytes[st] > 0:
            rec_k["event_hbm_frac"] = sbytes[st] / (stage_ms[st] * 1e-3) / PEAK_HBM
        if st in traced:
            rec_k["rocprof_us"] = traced[st]
            if sbytes[st] > 0 and traced[st] > 0:
                rec_k["rocprof_hbm_frac"] = sbytes[st] / (traced[st] * 1e-6) / PEAK_HBM
        kernels[STAGE_KERNEL[st]] = rec_k
    dom = max((st for st in STAGES if sbytes[st] > 0), key=lambda st: stage_ms[st])
    dom_achieved = sbytes[dom] / (stage_ms[dom] * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"nystrom_attention_forward_B{cfg.B}_H{cfg.H}_n{cfg.n}_"
                               f"d{cfg.d}_m{cfg.m}_conv{cfg.conv_width}_iters{cfg.pinv_iters}"
                               + ("_ragged" if lengths else ""),
                   "name": name,
                   "B": cfg.B, "H": cfg.H, "n": cfg.n, "d": cfg.d, "m": cfg.m,
                   "conv_width": cfg.conv_width, "pinv_iters": cfg.pinv_iters,
                   "inputs": "two alternating seeded N(0,1) sets",
                   **({"lengths": lengths} if lengths else {})},
        "roofline": roof,
        "dominant_kernel": {"kernel": STAGE_KERNEL[dom], "bound": "hbm",
                            "achieved": dom_achieved, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                            "frac": dom_achieved * 1e9 / PEAK_HBM,
                            "timing": "HIP event interval on the forward's stream",
                            "traffic": None if lengths else measured_traffic(dom, name)},
        "kernels": kernels,
        "clock_ramp": ramp,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, sets[0], budget_s=args.cpu_budget,
                                           lengths=lengths)
        if args.cpu_1thread:
            rec["cpu_baseline_1thread"] = cpu_baseline(cfg, sets[0], budget_s=5.0,
                                                       lengths=lengths, threads=1)
    att.close()
    print(json.dumps(rec), flush=True)


def backward_bench(args, cfg):
    """Steps of the backward pass on the workload: one nys_attn_backward call per step
    (it recomputes the landmarks and the context states, then the gradient kernels),
    inputs and dout resident, two alternating seeded sets."""
    import torch
    from efficient_transformer_attention_segment_amd import NystromAttention
    from efficient_transformer_attention_segment_amd import inputs as gen
    sets = [gen.make_inputs(cfg), gen.make_inputs(cfg, seed=cfg.seed + 1000)]

    def dev(a):
        if cfg.dtype == gen.BF16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    rng = np.random.default_rng(cfg.seed + 555)

    def draw():
        g = rng.standard_normal((cfg.B, cfg.H, cfg.n, cfg.d), dtype=np.float32)
        return gen.f32_to_bf16_bits(g) if cfg.dtype == gen.BF16 else g

    gs = [dev(draw()) for _ in sets]
    dev_sets = [(dev(s.q_dev), dev(s.k_dev), dev(s.v_dev), torch.from_numpy(s.w).cuda())
                for s in sets]
    att = NystromAttention(cfg.B, cfg.H, cfg.n, cfg.d, cfg.m, cfg.conv_width,
                           cfg.pinv_iters, cfg.dtype)

    def step(i):
        q, k, v, w = dev_sets[i % 2]
        att.backward(q, k, v, w, gs[i % 2])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for i in range(args.steps):
        step(i)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    e = 2 if cfg.dtype == gen.BF16 else 4
    compulsory = 7 * cfg.bh * cfg.n * cfg.d * e   # read Q, K, V, dO; write dQ, dK, dV
    general = cfg.dtype != gen.BF16 or cfg.m > 64
    roof_ms = compulsory / (HBM_PEAK_GBS * 1e9) * 1e3
    rec = {
        "metric": "Nystrom attn backward tokens/s",
        "value": cfg.tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"nystrom_attention_backward_B{cfg.B}_H{cfg.H}_n{cfg.n}_"
                               f"d{cfg.d}_m{cfg.m}_conv{cfg.conv_width}_iters{cfg.pinv_iters}",
                   "B": cfg.B, "H": cfg.H, "n": cfg.n, "d": cfg.d, "m": cfg.m,
                   "path": "general (batched fp32 products)" if general else "fused kernels",
                   "inputs": "two alternating seeded N(0,1) sets, dout N(0,1)"},
        "path_roofline": {"bound": "hbm", "compulsory_bytes": compulsory,
                          "roofline_ms": roof_ms, "frac": roof_ms / ms},
    }
    att.close()
    print(json.dumps(rec), flush=True)


def flash_bench(args, cfg):
    """Steps of FLASH mixed-chunk attention on the workload's Q, K, V: the chunk-state
    phase (K^T V per chunk, global sums) and the attention phase, each timed with events
    on the stream they run on."""
    import torch
    from efficient_transformer_attention_segment_amd import (nys_flash_attend, nys_flash_states,
                                                             nys_flash_workspace_bytes)
    from efficient_transformer_attention_segment_amd import inputs as gen
    c, causal = args.flash, args.causal
    B, H, n, d = cfg.B, cfg.H, cfg.n, cfg.d
    sets = [gen.make_inputs(cfg), gen.make_inputs(cfg, seed=cfg.seed + 1000)]

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    dev_sets = [(dev(s.q_dev), dev(s.k_dev), dev(s.v_dev)) for s in sets]
    outs = [torch.empty_like(dev_sets[0][0]) for _ in sets]
    nb = nys_flash_workspace_bytes(B, H, n, d, c, causal)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def states(i):
        _, k, v = dev_sets[i % 2]
        nys_flash_states(k.data_ptr(), v.data_ptr(), B, H, n, d, c, causal, ws.data_ptr(), nb,
                         stream)

    def attend(i):
        q, k, v = dev_sets[i % 2]
        nys_flash_attend(q.data_ptr(), k.data_ptr(), v.data_ptr(), outs[i % 2].data_ptr(), B, H,
                         n, d, c, causal, ws.data_ptr(), nb, stream)

    for i in range(args.warmup):
        states(i)
        attend(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for i in range(args.steps):
        states(i)
        attend(i)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    nprof = min(args.steps, 200)
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nprof)]
    for i in range(nprof):
        marks[i][0].record()
        states(i)
        marks[i][1].record()
        attend(i)
        marks[i][2].record()
    torch.cuda.synchronize()
    st_ms = float(np.mean([m[0].elapsed_time(m[1]) for m in marks]))
    at_ms = float(np.mean([m[1].elapsed_time(m[2]) for m in marks]))
    e = 2
    attend_bytes = 4 * cfg.bh * n * d * e            # read Q, K, V; write out
    state_bytes = 2 * cfg.bh * n * d * e             # read K, V
    achieved = attend_bytes / (at_ms * 1e-3) / 1e9
    compulsory = 4 * cfg.bh * n * d * e
    rec = {
        "metric": "FLASH mixed-chunk attention fwd tokens/s",
        "value": cfg.tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"flash_mixed_chunk_B{B}_H{H}_n{n}_d{d}_chunk{c}_"
                               + ("causal" if causal else "bidirectional"),
                   "B": B, "H": H, "n": n, "d": d, "chunk": c, "causal": causal,
                   "inputs": "two alternating seeded N(0,1) sets"},
        "roofline": {"kernel": "flash_attend_kernel", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "algorithmic_bytes": attend_bytes, "traffic": None},
        "stages_ms": {"states": st_ms, "attend": at_ms},
        "state_roofline": {"bound": "hbm", "algorithmic_bytes": state_bytes,
                           "achieved": state_bytes / (st_ms * 1e-3) / 1e9},
        "path_roofline": {"bound": "hbm", "compulsory_bytes": compulsory,
                          "roofline_ms": compulsory / (HBM_PEAK_GBS * 1e9) * 1e3,
                          "frac": compulsory / (HBM_PEAK_GBS * 1e9) * 1e3 / ms},
    }
    if not args.no_cpu_baseline:
        import time
        import oracle
        heads, t0 = [], time.perf_counter()
        while time.perf_counter() - t0 < 10.0 and len(heads) < cfg.bh:
            pair = (len(heads) // H, len(heads) % H)
            oracle.mixed_chunk_attention(sets[0].q, sets[0].k, sets[0].v, c, causal, heads=[pair])
            heads.append(pair)
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": len(heads) * n / dt, "unit": "tokens/s",
                               "cores": os.cpu_count() or 1, "kind": "oracle",
                               "sample": f"{len(heads)} of {cfg.bh} heads in {dt:.1f} s"}
    print(json.dumps(rec), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def proj_roofline(flops: float, nbytes: float, ms: float) -> dict:
    """Roofline of one projection GEMM: whichever of dense bf16 MFMA and HBM takes
    longer at peak binds."""
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    if t_mfma >= t_hbm:
        a = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": a, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": a / MFMA_BF16_PEAK_TFLOPS}
    a = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": a / HBM_PEAK_GBS}


def layer_bench(args, cfg):
    """Steps of the projected layer: x [B n][D] -> Q, K, V (bf16 GEMM) -> Nystrom
    forward -> output projection -> y [B n][D]. Per-kernel times come from torch events
    on the stream the projections are launched on (torch's current stream) and from the
    library's own stage events for the core."""
    import torch
    from efficient_transformer_attention_segment_amd import NystromLayer, nys_proj_out, nys_proj_qkv
    from efficient_transformer_attention_segment_amd import inputs as gen
    D = args.layer
    sets = [gen.make_layer_inputs(cfg, D), gen.make_layer_inputs(cfg, D, seed=cfg.seed + 1000)]

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    dev_sets = [(dev(s.x_dev), dev(s.w_qkv_dev), dev(s.w_o_dev), torch.from_numpy(s.w).cuda())
                for s in sets]
    ys = [torch.empty(cfg.B, cfg.n, D, dtype=torch.bfloat16, device="cuda") for _ in sets]
    layer = NystromLayer(cfg.B, cfg.H, cfg.n, cfg.d, cfg.m, D, cfg.conv_width, cfg.pinv_iters)

    def step(i):
        x, wq, wo, w = dev_sets[i % 2]
        layer.forward(x, wq, wo, w, y=ys[i % 2])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for i in range(args.steps):
        step(i)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / args.steps

    # per-kernel times: the projections bracketed by events on their own stream, the core
    # by the library's stage events, over a shorter profiled pass
    nprof = min(args.steps, 200)
    B, H, n, d = cfg.B, cfg.H, cfg.n, cfg.d
    stream = torch.cuda.current_stream().cuda_stream
    buf = layer._buffers(torch.device("cuda", 0))
    q, k, v, o = buf[0], buf[1], buf[2], buf[3]
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nprof)]
    layer.attn.profile_enable(nprof)
    for i in range(nprof):
        x, wq, wo, w = dev_sets[i % 2]
        e = marks[i]
        e[0].record()
        nys_proj_qkv(x.data_ptr(), wq.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                     B, H, n, d, D, stream)
        e[1].record()
        layer.attn.forward(q, k, v, w, out=o)
        e[2].record()
        nys_proj_out(o.data_ptr(), wo.data_ptr(), ys[i % 2].data_ptr(), B, H, n, d, D, stream)
        e[3].record()
    torch.cuda.synchronize()
    qkv_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in marks]))
    out_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in marks]))
    prof = np.array(layer.attn.profile_read(nprof), dtype=np.float64)
    stage_ms = {s: float(prof[:, j].mean()) for j, s in enumerate(STAGES)}
    stage_ms["qkv_proj"], stage_ms["out_proj"] = qkv_ms, out_ms

    M, HD = B * n, H * d
    qkv_flops, out_flops = 2.0 * M * 3 * HD * D, 2.0 * M * D * HD
    qkv_bytes = 2.0 * (M * D + 3 * HD * D + 3 * M * HD)   # read x, w_qkv; write q, k, v
    out_bytes = 2.0 * (M * HD + D * HD + M * D)           # read o, w_o; write y
    qkv_roof = proj_roofline(qkv_flops, qkv_bytes, qkv_ms)
    out_roof = proj_roofline(out_flops, out_bytes, out_ms)
    value = cfg.tokens / (ms * 1e-3)
    rec = {
        "metric": "Nystrom layer (projections + attention) fwd tokens/s",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"nystrom_layer_B{B}_H{H}_n{n}_d{d}_m{cfg.m}_D{D}_"
                               f"conv{cfg.conv_width}_iters{cfg.pinv_iters}",
                   "B": B, "H": H, "n": n, "d": d, "m": cfg.m, "d_model": D,
                   "inputs": "two alternating seeded sets: x ~ N(0,1), weights ~ "
                             "N(0, 1/fan_in)"},
        "roofline": {"kernel": "qkv_proj_kernel", **qkv_roof,
                     "flops": qkv_flops, "algorithmic_bytes": qkv_bytes, "traffic": None},
        "out_proj_roofline": {"kernel": "out_proj_kernel", **out_roof,
                              "flops": out_flops, "algorithmic_bytes": out_bytes},
        "stages_ms": stage_ms,
    }
    layer.close()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
