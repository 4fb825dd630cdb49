"""Throughput of the segment-causal joint attention hot path on one MI355X.

One step = one segment of one DiT layer: the 8 denoising layer-steps of the
distilled sampler (each: RoPE of the current video Q and K, then joint
attention over the INT8 history plus the current segment), then the window
select and the INT8 append of the segment's K/V to the cache. Inputs are
seeded synthetic tensors at the workload's shapes, resident in HBM before the
timed region. Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--config c4] [--no-cpu-baseline]
  python bench.py --train [--steps K] [--warmup W]   (packed training form:
      forward + backward of one layer's attention over 346,528 packed rows)
  python bench.py --archive [--steps K] [--warmup W] (CPU history archive:
      window fetch and segment store over PCIe, overlap with attention)
  python bench.py --linear [--steps K] [--warmup W]  (INT8-weight linears of
      one block's video stream at 63,360 rows)
  python bench.py --camera [--steps K] [--warmup W]  (camera cross-attention
      of c4's video rows)
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from workloads import HEAD_DIM  # noqa: E402

METRIC = "attention TFLOP/s + video tokens/s per layer-step; % of MFMA/HBM roofline"
DENOISE_STEPS = 8            # distilled sampler steps per segment
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
ATTN_KERNEL = "attn_kernel"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bwd_source_hash():
    with open(os.path.join(ROOT, "segment_causal_dit_amd", "csrc", "attn_bwd.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def attn_source_hash():
    with open(os.path.join(ROOT, "segment_causal_dit_amd", "csrc", "attn.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def history_path(cfg, int8_attn="window"):
    """How the attention reads the history in this run (the counter summary
    is only valid for the same path)."""
    if not len(cfg.hist_t):
        return "none"
    if cfg.cache_dtype == "int8":
        return "int8 window expanded to bf16" if int8_attn == "window" else "int8 cache"
    return "bf16 cache"


def measured_traffic(cfg, path):
    """HBM bytes per attention launch from the committed counter summary, or
    None when it is missing or was taken on a different kernel source or
    history path."""
    try:
        with open(os.path.join(ROOT, "profiles", "attn_%s_counters.json" % cfg.name)) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    if (s.get("attn_source_sha") != attn_source_hash() or s.get("workload") != cfg.name
            or s.get("history_path") != path):
        return None
    return s.get("hbm_bytes_per_launch")


def cpu_model():
    """The host CPU's model name (for the CPU baseline's context)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def config_rates(names, reps=20):
    """Attention at the shorter configurations, timed like the main line: the
    history appended through the library (INT8 windows expanded to bf16 once,
    as in the step), then `reps` attention launches timed with HIP events on
    the launch stream. Returns {name: {...}} with each one's own roofline
    fraction."""
    import torch
    import segment_causal_dit_amd as sc
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    out = {}

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    for name in names:
        cfg = workloads.CONFIGS[name]
        inp = workloads.make_inputs(cfg)
        q, k, v = bf(inp.q), bf(inp.k), bf(inp.v)
        tl = cfg.segments[0].text_len
        pos = torch.from_numpy(inp.pos).to(dev)
        sc.rope3d_apply(q[tl:], pos)
        sc.rope3d_apply(k[tl:], pos)
        cache = hist = None
        deq_ms = None
        if len(cfg.hist_t):
            cache = sc.KVCache(cfg.n_slots, cfg.n_heads, cfg.tokens_per_frame, cfg.cache_dtype, dev)
            hk = bf(inp.hist_k)
            sc.rope3d_apply(hk, torch.from_numpy(inp.hist_pos).to(dev))
            sc.kv_cache_append(cache, 0, hk, bf(inp.hist_v))
            cache.slot_t[:] = inp.slot_t
            hist = torch.from_numpy(sc.window_select(cache.slot_t, cfg.window)).to(dev)
            if cfg.cache_dtype == "int8":
                win = sc.KVCache(len(hist), cfg.n_heads, cfg.tokens_per_frame, "bf16", dev)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                sc.kv_window_dequant(cache, hist, win)
                a.record(stream)
                sc.kv_window_dequant(cache, hist, win)
                b.record(stream)
                torch.cuda.synchronize()
                deq_ms = a.elapsed_time(b)
                cache, hist = win, torch.arange(len(hist), dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        ws = attn_workspace(sc, cfg.n_cur, cfg.n_heads, inp.segments, hist, cache, dev)

        def call():
            sc.segcausal_joint_attn(q, k, v, inp.segments, cfg.sm_scale, cache=cache, hist_slots=hist, out=o,
                                    workspace=ws)

        for _ in range(3):
            call()
        torch.cuda.synchronize()
        evs = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            call()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in evs)
        med = ms[len(ms) // 2]
        tflops = cfg.flops() / (med * 1e-3) / 1e12
        out[name] = {"attn_ms_median": round(med, 4), "attn_ms_min": round(ms[0], 4),
                     "tflops": round(tflops, 2), "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "window_dequant_ms": round(deq_ms, 4) if deq_ms is not None else None,
                     "n_cur": cfg.n_cur, "n_hist_keys": cfg.n_hist_rows, "cache": cfg.cache_dtype
                     if len(cfg.hist_t) else None}
        log("%s: attention %.4f ms (median of %d), %.1f TFLOP/s, %.1f%% of bf16 peak"
            % (name, med, reps, tflops, 100 * tflops / PEAK_BF16_TFLOPS))
        del q, k, v, o, cache, hist
        torch.cuda.empty_cache()
    return out


def attn_workspace(sc, n_cur, n_heads, segments, hist, cache, dev):
    """The attention's split workspace, allocated once outside the timed
    region (None when the call would not split)."""
    import torch
    n_hist = 0 if hist is None else int(hist.numel())
    need = sc.attn_workspace_bytes(n_cur, n_heads, segments, n_hist, cache if n_hist else None)
    return torch.empty(need, dtype=torch.uint8, device=dev) if need > 0 else None


def cpu_baseline(cfg, inp, n_rows=512):
    """The fp64 oracle's attention on a bounded sample of the workload: all
    heads of n_rows random query rows against every key. History codes are
    drawn directly (seeded), so no GPU result feeds the oracle."""
    import oracle
    h = cfg.n_heads
    rng = np.random.default_rng(1234)
    nf = cfg.window
    kc, vc, ks, vs = workloads.uniform_int8_cache(cfg, nf)
    hk, hv = oracle.history_keys(kc, vc, np.arange(nf), ks, vs)
    del kc, vc
    q, k, v = (oracle.bf16_bits_to_f64(x) for x in (inp.q, inp.k, inp.v))
    rows = np.sort(rng.choice(cfg.n_cur, n_rows, replace=False))
    segs = [oracle.Segment(*s) for s in inp.segments]
    cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    oracle.joint_attn_rows(q, k, v, segs, rows, hk, hv, cfg.sm_scale, chunk=256, workers=cores)
    dt = time.perf_counter() - t0
    flops = 4 * HEAD_DIM * h * n_rows * (cfg.n_hist_rows + cfg.n_cur)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "attention of %d random query rows x %d heads over all %d keys "
                      "(numpy float64, %d threads, %.1f s)"
                      % (n_rows, h, cfg.n_hist_rows + cfg.n_cur, cores, dt)}


COPY_BYTES = 1 << 31         # calibration copy for the HBM byte counters


def counters_workload(cfg_name):
    """Workload for rocprofv3 --pmc passes: one plain device copy of
    COPY_BYTES (calibrates FETCH_SIZE/WRITE_SIZE against known traffic), then
    one attention call on the workload."""
    import torch
    import segment_causal_dit_amd as sc
    cfg = workloads.CONFIGS[cfg_name]
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    inp = workloads.make_inputs(cfg)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = bf(inp.q), bf(inp.k), bf(inp.v)
    cache, hist = None, None
    if len(cfg.hist_t):
        cache = sc.KVCache(cfg.n_slots, cfg.n_heads, cfg.tokens_per_frame, cfg.cache_dtype, dev)
        hk = bf(inp.hist_k)
        sc.rope3d_apply(hk, torch.from_numpy(inp.hist_pos).to(dev))
        sc.kv_cache_append(cache, 0, hk, bf(inp.hist_v))
        cache.slot_t[:] = inp.slot_t
        hist = torch.from_numpy(sc.window_select(cache.slot_t, cfg.window)).to(dev)
        if cfg.cache_dtype == "int8":       # the bench's path: expand the window, attend over bf16
            win = sc.KVCache(len(hist), cfg.n_heads, cfg.tokens_per_frame, "bf16", dev)
            sc.kv_window_dequant(cache, hist, win)
            cache, hist = win, torch.arange(len(hist), dtype=torch.int32, device=dev)
    ws = attn_workspace(sc, cfg.n_cur, cfg.n_heads, inp.segments, hist, cache, dev)
    torch.cuda.synchronize()
    sc.segcausal_joint_attn(q, k, v, inp.segments, cfg.sm_scale, cache=cache, hist_slots=hist, workspace=ws)
    torch.cuda.synchronize()
    log("counters workload done")


DRAM_READ, DRAM_WRITE = "TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"
# counter passes profile only the attention and the calibration copy
KERNEL_FILTER = "--kernel-include-regex 'attn_kernel|elementwise|copy'"


def summarize_counters(cfg_name, fetch_dir, write_dir, out_path, dram_dir=None):
    """Turn two rocprofv3 --pmc CSV outputs (FETCH_SIZE, WRITE_SIZE) into HBM
    bytes per attention launch, scaled by the calibration copy; with a third
    (the L2's 32-byte read and write requests to the memory controller), the
    same from those counters beside it."""
    import csv
    import glob

    def read(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Dispatch_Id"], r["Kernel_Name"])
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        copy = [v for (i, n), v in vals.items() if "copy" in n.lower() or "elementwise" in n.lower()]
        attn = [v for (i, n), v in vals.items() if ATTN_KERNEL in n]
        return max(copy), attn
    f_copy, f_attn = read(fetch_dir, "FETCH_SIZE")
    w_copy, w_attn = read(write_dir, "WRITE_SIZE")
    f_scale = COPY_BYTES / 1024.0 / f_copy      # counters are KiB
    w_scale = COPY_BYTES / 1024.0 / w_copy
    fetch = float(np.mean(f_attn)) * 1024.0 * f_scale
    write = float(np.mean(w_attn)) * 1024.0 * w_scale
    dram = None
    if dram_dir:
        r_copy, r_attn = read(dram_dir, DRAM_READ)
        x_copy, x_attn = read(dram_dir, DRAM_WRITE)
        dram = {"read_bytes_per_launch": float(np.mean(r_attn)) * 32.0,
                "write_bytes_per_launch": float(np.mean(x_attn)) * 32.0,
                "calibration": {"copy_bytes": COPY_BYTES, "read_bytes_counted": r_copy * 32.0,
                                "write_bytes_counted": x_copy * 32.0,
                                "read_ratio": r_copy * 32.0 / COPY_BYTES,
                                "write_ratio": x_copy * 32.0 / COPY_BYTES},
                "counters": [DRAM_READ, DRAM_WRITE]}
    summary = {
        "workload": cfg_name, "kernel": ATTN_KERNEL, "attn_source_sha": attn_source_hash(),
        "history_path": history_path(workloads.CONFIGS[cfg_name]),
        "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
        "hbm_bytes_per_launch": fetch + write,
        "calibration": {"copy_bytes": COPY_BYTES, "fetch_kib_read": f_copy,
                        "write_kib_read": w_copy, "fetch_scale": f_scale, "write_scale": w_scale},
        "dram_requests": dram,
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE %s --output-format csv -d <fetch_dir> -- "
            "python3 bench.py --config %s --counters-workload" % (KERNEL_FILTER, cfg_name),
            "rocprofv3 --pmc WRITE_SIZE %s --output-format csv -d <write_dir> -- "
            "python3 bench.py --config %s --counters-workload" % (KERNEL_FILTER, cfg_name),
            "rocprofv3 --pmc %s %s %s --output-format csv -d <dram_dir> -- "
            "python3 bench.py --config %s --counters-workload" % (DRAM_READ, DRAM_WRITE, KERNEL_FILTER, cfg_name),
            "python3 bench.py --config %s --summarize-counters <fetch_dir> <write_dir> [<dram_dir>]"
            % cfg_name],
    }
    with open(out_path, "w") as f:
        json.dump(summary, f, indent=1)
    print(json.dumps(summary))


ISSUE_COUNTERS = ("SQ_WAVES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES "
                  "SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_SALU GRBM_GUI_ACTIVE")
N_XCD, N_SIMD = 8, 1024      # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def summarize_issue(cfg_name, issue_dir, out_path, kernel=ATTN_KERNEL, workload_cmd=None):
    """Per-SIMD issue figures of the attention launch from one rocprofv3 --pmc
    pass over ISSUE_COUNTERS (counters summed over the chip by rocprofv3):
    active cycles per XCD = GRBM_GUI_ACTIVE / 8 (their ratio to the dispatch's
    duration is the average clock); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024
    SIMDs over those cycles (32 per 32x32x16 bf16 MFMA); coexec the same for
    SQ_VALU_MFMA_COEXEC_CYCLES; VALU active = 4 x SQ_ACTIVE_INST_VALU (counted
    in quad-cycles) over the SIMD-cycles; instruction mix per MFMA."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(issue_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if kernel not in r["Kernel_Name"]:
                continue
            d = per.setdefault(r["Dispatch_Id"], {"_dur": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit("no %s dispatch in %s" % (kernel, issue_dir))
    launches = []
    for d in per.values():
        cyc = d["GRBM_GUI_ACTIVE"] / N_XCD
        mfma = d["SQ_INSTS_MFMA"]
        launches.append({
            "duration_ms": d["_dur"] * 1e3, "clock_ghz": cyc / d["_dur"] * 1e-9,
            "waves": d["SQ_WAVES"], "mfma_insts": mfma,
            "mfma_busy_frac": d["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / cyc,
            "mfma_busy_cycles_per_mfma": d["SQ_VALU_MFMA_BUSY_CYCLES"] / mfma,
            "valu_mfma_coexec_frac": d["SQ_VALU_MFMA_COEXEC_CYCLES"] / N_SIMD / cyc,
            "valu_active_frac": 4.0 * d["SQ_ACTIVE_INST_VALU"] / N_SIMD / cyc,
            "valu_insts_per_mfma": (d["SQ_INSTS_VALU"] - mfma) / mfma,
            "salu_insts_per_mfma": d["SQ_INSTS_SALU"] / mfma,
        })
    keys = [k for k in launches[0]]
    mean = {k: float(np.mean([x[k] for x in launches])) for k in keys}
    if workload_cmd is None:
        workload_cmd = "python3 bench.py --config %s --counters-workload" % cfg_name
        summarize_cmd = "python3 bench.py --config %s --summarize-issue <issue_dir>" % cfg_name
        filt = KERNEL_FILTER
    else:
        summarize_cmd = "python3 bench.py --train --summarize-issue <issue_dir> --issue-kernel %s" % kernel
        filt = "--kernel-include-regex %s" % kernel
    summary = {
        "workload": cfg_name, "kernel": kernel,
        "source_sha": attn_source_hash() if kernel == ATTN_KERNEL else bwd_source_hash(),
        "history_path": history_path(workloads.CONFIGS[cfg_name]) if cfg_name in workloads.CONFIGS else None,
        "launches": len(launches), "mean": mean,
        "command": "rocprofv3 --pmc %s %s --output-format csv -d <issue_dir> -- %s; %s"
                   % (ISSUE_COUNTERS, filt, workload_cmd, summarize_cmd),
    }
    with open(out_path, "w") as f:
        json.dump(summary, f, indent=1)
    print(json.dumps(summary))


TRAIN_METRIC = "packed-form attention forward+backward TFLOP/s; % of bf16 MFMA roofline"


def cpu_baseline_train(cfg, n_rows=16384):
    """The fp64 oracle's gradients (which recompute the forward) on a bounded
    sample of the packed workload: one head, the first n_rows rows of the
    first segment (a packed sequence of its own)."""
    import oracle
    seg0 = cfg.segments[0]
    shape = (n_rows, 1, HEAD_DIM)
    q = oracle.bf16_bits_to_f64(workloads.normal_bf16(0, shape, cfg.q_scale))
    k, v, do = (oracle.bf16_bits_to_f64(workloads.normal_bf16(i, shape)) for i in (1, 2, 7))
    segs = [oracle.Segment(0, seg0.text_len, seg0.text_valid)]
    pairs = n_rows * (n_rows - (seg0.text_len - seg0.text_valid))
    t0 = time.perf_counter()
    oracle.joint_attn_backward(q, k, v, segs, do, sm_scale=cfg.sm_scale)
    dt = time.perf_counter() - t0
    flops = 14 * HEAD_DIM * pairs
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": os.cpu_count() or 1,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "forward+backward of the first %d rows of one segment, 1 head "
                      "(numpy float64, %.1f s)" % (n_rows, dt)}


def train_bench(args):
    """Packed training form: one step = the forward (with lse) and the
    backward of one layer's segment-causal attention over the packed
    sequence (q and k rotated once, outside the timed region)."""
    import torch
    import segment_causal_dit_amd as sc

    cfg = workloads.TRAIN["train13"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    h = cfg.n_heads
    log("generating %s inputs" % cfg.name)
    inp = workloads.make_inputs(cfg)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = bf(inp.q), bf(inp.k), bf(inp.v)
    do = bf(workloads.upstream_grad(cfg))
    pos = torch.from_numpy(inp.pos).to(dev)
    pr = 0
    g = cfg.tokens_per_frame
    for (start, tl, _), sg in zip(inp.segments, cfg.segments):
        n = sg.n_frames * g
        sc.rope3d_apply(q[start + tl:start + tl + n], pos[pr:pr + n])
        sc.rope3d_apply(k[start + tl:start + tl + n], pos[pr:pr + n])
        pr += n
    segs = inp.segments
    o = torch.empty_like(q)
    lse = torch.empty((h, cfg.n_cur), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    delta = torch.empty_like(lse)
    stream = torch.cuda.current_stream()
    ev = {"fwd": [], "bwd": []}

    def rec(name, fn):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        ev[name].append((a, b))

    def one_step():
        rec("fwd", lambda: sc.segcausal_joint_attn(q, k, v, segs, cfg.sm_scale, out=o, lse=lse))
        rec("bwd", lambda: sc.segcausal_joint_attn_bwd(q, k, v, o, do, lse, segs, cfg.sm_scale,
                                                       dq=dq, dk=dk, dv=dv, delta=delta))

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    for k_ in ev:
        ev[k_].clear()
    log("timing %d steps" % args.steps)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        one_step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    fwd_ms = float(np.mean([a.elapsed_time(b) for a, b in ev["fwd"]]))
    bwd_ms = float(np.mean([a.elapsed_time(b) for a, b in ev["bwd"]]))
    pairs = cfg.visible_pairs() * h
    fwd_flops, bwd_flops = 4 * HEAD_DIM * pairs, 10 * HEAD_DIM * pairs
    step_tflops = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12
    bwd_tflops = bwd_flops / (bwd_ms * 1e-3) / 1e12
    fwd_tflops = fwd_flops / (fwd_ms * 1e-3) / 1e12
    log("forward %.2f ms (%.1f%% of bf16 peak)  backward %.2f ms (%.1f%%)  step %.2f ms"
        % (fwd_ms, 100 * fwd_tflops / PEAK_BF16_TFLOPS, bwd_ms, 100 * bwd_tflops / PEAK_BF16_TFLOPS,
           ms_step))
    line = {
        "metric": TRAIN_METRIC,
        "value": round(step_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "%s: packed sequence of %d segments x (256 text + 30 frames of 22x40) = %d "
                        "rows x %d heads x 128, no cache; forward (with lse) + backward "
                        "(delta, dQ, dK/dV) of one layer's attention" % (cfg.name, len(cfg.segments),
                                                                        cfg.n_cur, h),
            "n_rows": cfg.n_cur, "segments": len(cfg.segments), "heads": h, "head_dim": HEAD_DIM,
        },
        "kernels_ms": {"forward": round(fwd_ms, 3), "backward": round(bwd_ms, 3)},
        "flops_per_visible_pair": {"forward": 4 * HEAD_DIM, "backward": 10 * HEAD_DIM},
        "roofline": {"bound": "mfma", "achieved": round(bwd_tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "backward call (delta + dQ + dK/dV)"},
        "forward_roofline_frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle sample)")
        line["cpu_baseline"] = cpu_baseline_train(cfg)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


ARCHIVE_METRIC = "history archive fetch GB/s (pinned host -> device frames); overlap with attention"
PEAK_PCIE_GBS = 64.0         # MI355X host link: PCIe Gen5 x16, per direction


def archive_bench(args):
    """CPU history archive on the full frame geometry (16 heads x 880 tokens,
    INT8 codes + fp32 scales, 3.72 MB per frame and layer): the fetch of an
    18-frame window from pinned host memory, the store of one 8-frame
    segment, and the fetch on a copy stream while the c3 attention (18 INT8
    history frames + an 8-frame segment) runs on the main stream."""
    import torch
    import segment_causal_dit_amd as sc

    cfg = workloads.CONFIGS["c3"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    h, g = cfg.n_heads, cfg.tokens_per_frame
    window, seg_frames, n_arch = 18, 8, 72
    frame_bytes = 2 * h * g * (HEAD_DIM + 4)
    arch = sc.KVCache.archive(n_arch, h, g, "int8")
    kc, vc, ks, vs = workloads.uniform_int8_cache(cfg, n_arch)
    for t, a in zip((arch.k, arch.v, arch.k_scale, arch.v_scale), (kc, vc, ks, vs)):
        t.copy_(torch.from_numpy(a))
    del kc, vc, ks, vs
    cache = sc.KVCache(cfg.n_slots + window, h, g, "int8", dev)
    inp = workloads.make_inputs(cfg)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = bf(inp.q), bf(inp.k), bf(inp.v)
    sc.kv_archive_fetch(arch, list(range(window)), cache, list(range(window)))
    hist = torch.arange(window, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    seg = cfg.segments[0]
    segs = [(0, seg.text_len, seg.text_valid)]
    copy_stream = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    fetch_frames = list(range(30, 30 + window))            # older frames, re-entering the window
    fetch_slots = list(range(cfg.n_slots, cfg.n_slots + window))
    store_slots = list(range(seg_frames))
    store_frames = list(range(n_arch - seg_frames, n_arch))

    def timed(fn, stream):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        return a, b

    ws = attn_workspace(sc, cfg.n_cur, cfg.n_heads, segs, hist, cache, dev)

    def attn():
        sc.segcausal_joint_attn(q, k, v, segs, cfg.sm_scale, cache=cache, hist_slots=hist, out=out,
                                workspace=ws)

    def fetch():
        sc.kv_archive_fetch(arch, fetch_frames, cache, fetch_slots, stream=copy_stream)

    def store():
        sc.kv_archive_store(cache, store_slots, arch, store_frames, stream=copy_stream)

    for _ in range(args.warmup):
        attn()
        fetch()
        store()
    torch.cuda.synchronize()
    res = {"fetch": [], "store": [], "attn": [], "attn_overlap": [], "fetch_overlap": []}
    for _ in range(args.steps):
        ev = timed(fetch, copy_stream)
        torch.cuda.synchronize()
        res["fetch"].append(ev[0].elapsed_time(ev[1]))
        ev = timed(store, copy_stream)
        torch.cuda.synchronize()
        res["store"].append(ev[0].elapsed_time(ev[1]))
        ev = timed(attn, main)
        torch.cuda.synchronize()
        res["attn"].append(ev[0].elapsed_time(ev[1]))
        # both at once: the copy stream starts when the attention does
        copy_stream.wait_stream(main)
        ea = timed(attn, main)
        ef = timed(fetch, copy_stream)
        torch.cuda.synchronize()
        res["attn_overlap"].append(ea[0].elapsed_time(ea[1]))
        res["fetch_overlap"].append(ef[0].elapsed_time(ef[1]))
    med = {k_: float(np.median(v_)) for k_, v_ in res.items()}
    fetch_bytes, store_bytes = window * frame_bytes, seg_frames * frame_bytes
    fetch_gbs = fetch_bytes / (med["fetch"] * 1e-3) / 1e9
    store_gbs = store_bytes / (med["store"] * 1e-3) / 1e9
    log("fetch %d frames %.3f ms (%.1f GB/s)  store %d frames %.3f ms (%.1f GB/s)  attention %.3f ms, "
        "with a concurrent fetch %.3f ms (fetch %.3f ms)" % (window, med["fetch"], fetch_gbs, seg_frames,
                                                              med["store"], store_gbs, med["attn"],
                                                              med["attn_overlap"], med["fetch_overlap"]))
    line = {
        "metric": ARCHIVE_METRIC,
        "value": round(fetch_gbs, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med["fetch"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": "archive: %d-frame INT8 window of 16 heads x 880 tokens (codes + fp32 scales, "
                               "%.2f MB per frame and layer) fetched from pinned host memory; store of an "
                               "%d-frame segment; fetch overlapped with the c3 attention (18 INT8 history "
                               "frames + 8-frame segment)" % (window, frame_bytes / 1e6, seg_frames)},
        "store_gbs": round(store_gbs, 3),
        "kernels_ms": {"fetch": round(med["fetch"], 4), "store": round(med["store"], 4),
                       "attention": round(med["attn"], 4),
                       "attention_with_concurrent_fetch": round(med["attn_overlap"], 4),
                       "fetch_concurrent_with_attention": round(med["fetch_overlap"], 4)},
        "roofline": {"bound": "pcie", "achieved": round(fetch_gbs, 3), "peak": PEAK_PCIE_GBS, "unit": "GB/s",
                     "frac": round(fetch_gbs / PEAK_PCIE_GBS, 4), "traffic": None,
                     "kernel": "host-to-device DMA of the window"},
    }
    if not args.no_cpu_baseline:
        import oracle
        a_np = arch.k.numpy()
        dst = np.zeros((window,) + a_np.shape[1:], a_np.dtype)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 10.0:
            for t in (arch.k, arch.v, arch.k_scale, arch.v_scale):
                a_ = t.numpy()
                oracle.move_frames(a_, fetch_frames, np.zeros((window,) + a_.shape[1:], a_.dtype),
                                   list(range(window)))
            reps += 1
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(reps * fetch_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                                "cpu_model": cpu_model(), "kind": "oracle",
                                "sample": "the oracle's indexed copy of the same %d frames in host memory, "
                                          "%d repetitions in %.1f s" % (window, reps, dt)}
        del dst
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


LINEAR_METRIC = "INT8-weight linear TFLOP/s over one block's video-stream linears (QKV, proj, MLP up, down)"


def linear_bench(args):
    """W8A16 linears of one double-stream block's video stream at c4's
    63,360 rows: QKV 2048 -> 6144, projection 2048 -> 2048, MLP 2048 -> 8192
    and 8192 -> 2048; one step = the four calls (code expansion + product)."""
    import torch
    import segment_causal_dit_amd as sc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ops = []
    for name, (m, n, k) in workloads.LINEARS.items():
        log("generating %s inputs" % name)
        x, codes, scale, bias = workloads.linear_inputs(m, n, k)
        ops.append(dict(name=name, m=m, n=n, k=k,
                        x=torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev),
                        w=torch.from_numpy(codes).to(dev), s=torch.from_numpy(scale).to(dev),
                        b=torch.from_numpy(bias).to(dev),
                        y=torch.empty((m, n), dtype=torch.bfloat16, device=dev),
                        ws=torch.empty(n * k, dtype=torch.bfloat16, device=dev), ev=[]))
    stream = torch.cuda.current_stream()

    def one_step():
        for o in ops:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            sc.w8a16_linear(o["x"], o["w"], o["s"], o["b"], out=o["y"], workspace=o["ws"])
            b.record(stream)
            o["ev"].append((a, b))

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    for o in ops:
        o["ev"].clear()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        one_step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    total_flops = sum(2 * o["m"] * o["n"] * o["k"] for o in ops)
    per = {}
    for o in ops:
        ms = float(np.mean([a.elapsed_time(b) for a, b in o["ev"]]))
        tf = 2 * o["m"] * o["n"] * o["k"] / (ms * 1e-3) / 1e12
        per[o["name"]] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        log("%-8s m=%d n=%d k=%d  %.3f ms  %.1f TFLOP/s (%.1f%% of bf16 peak)"
            % (o["name"], o["m"], o["n"], o["k"], ms, tf, 100 * tf / PEAK_BF16_TFLOPS))
    value = total_flops / (ms_step * 1e-3) / 1e12
    qkv = per["qkv"]
    line = {
        "metric": LINEAR_METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "linears: the video stream of one double-stream block at 63,360 rows (c4's "
                               "video tokens): QKV 2048->6144, proj 2048->2048, MLP 2048->8192, 8192->2048; "
                               "INT8 codes + per-channel fp32 scales, bf16 activations, fp32 bias"},
        "per_linear": per,
        "roofline": {"bound": "mfma", "achieved": qkv["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": qkv["frac"], "traffic": None,
                     "kernel": "QKV call (code expansion + product), 2 * 63,360 * 6,144 * 2,048 flops"},
    }
    if not args.no_cpu_baseline:
        import oracle
        del ops
        torch.cuda.empty_cache()
        dt, flops = 0.0, 0
        for name, (m, n, k) in workloads.LINEARS.items():
            x, codes, scale, bias = workloads.linear_inputs(m, n, k)
            xs = oracle.bf16_bits_to_f64(x)
            del x
            t = time.perf_counter()
            oracle.w8a16_linear(xs, codes, scale, bias)
            dt += time.perf_counter() - t
            flops += 2 * m * n * k
            del xs
        line["cpu_baseline"] = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
                                "cores": os.cpu_count() or 1, "cpu_model": cpu_model(), "kind": "oracle",
                                "sample": "all four linears at full size (numpy float64 matmul, %.1f s)" % dt}
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


CAMERA_METRIC = "camera cross-attention GB/s (video rows x heads over their latent frame's camera tokens)"


def camera_bench(args):
    """Camera cross-attention over c4's 63,360 video rows (72 latent frames of
    880 tokens, 16 heads): one camera token per latent frame (the pages'
    configuration: o = v of the frame, a pure write), and four tokens per frame
    through the general softmax path."""
    import torch
    import segment_causal_dit_amd as sc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = workloads.CONFIGS["c4"]
    n, h, tpc = cfg.n_video, cfg.n_heads, cfg.tokens_per_frame
    n_frames = n // tpc
    q = torch.from_numpy(workloads.normal_bf16(20, (n, h, HEAD_DIM)).view(np.int16)).view(torch.bfloat16).to(dev)
    res = {}
    for t_cam in (1, 4):
        k = torch.from_numpy(workloads.normal_bf16(21, (n_frames * t_cam, h, HEAD_DIM)).view(np.int16)).view(
            torch.bfloat16).to(dev)
        v = torch.from_numpy(workloads.normal_bf16(22, (n_frames * t_cam, h, HEAD_DIM)).view(np.int16)).view(
            torch.bfloat16).to(dev)
        o = torch.empty_like(q)
        for _ in range(args.warmup):
            sc.camera_cross_attn(q, k, v, tpc, 1.0 / math.sqrt(HEAD_DIM), out=o)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            sc.camera_cross_attn(q, k, v, tpc, 1.0 / math.sqrt(HEAD_DIM), out=o)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        byts = n * h * HEAD_DIM * 2 * (1 if t_cam == 1 else 2)      # o written (and q read)
        res[t_cam] = (ms, byts / (ms * 1e-3) / 1e9)
        log("t_cam %d: %.4f ms  %.0f GB/s (%.1f%% of HBM peak)" % (t_cam, ms, res[t_cam][1],
                                                                  100 * res[t_cam][1] / PEAK_HBM_GBS))
    ms1, gbs1 = res[1]
    line = {
        "metric": CAMERA_METRIC,
        "value": round(gbs1, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms1, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "camera: c4's 63,360 video rows (72 latent frames of 22x40) x 16 heads x 128, "
                               "one camera token per latent frame (o = v of the frame, 259.5 MB written); "
                               "four tokens per frame through the softmax path reported beside it"},
        "general_path_t_cam4": {"ms": round(res[4][0], 4), "gbs": round(res[4][1], 1),
                                "hbm_frac": round(res[4][1] / PEAK_HBM_GBS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(gbs1, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs1 / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "camera_attn_kernel, one camera token per frame: 256 B written per (row, head)"},
    }
    if not args.no_cpu_baseline:
        import oracle
        f = oracle.bf16_bits_to_f64
        rows = n                              # all 72 latent frames, four camera tokens each
        qs = f(workloads.normal_bf16(20, (n, h, HEAD_DIM)))
        ks = f(workloads.normal_bf16(21, (n_frames * 4, h, HEAD_DIM)))
        vs = f(workloads.normal_bf16(22, (n_frames * 4, h, HEAD_DIM)))
        t = time.perf_counter()
        oracle.camera_cross_attn(qs, ks, vs, tpc, 4, 1.0 / math.sqrt(HEAD_DIM))
        dt = time.perf_counter() - t
        line["cpu_baseline"] = {"value": round(rows * h * HEAD_DIM * 2 * 2 / dt / 1e9, 3), "unit": "GB/s",
                                "cores": 1, "cpu_model": cpu_model(), "kind": "oracle",
                                "sample": "the oracle's softmax path on all 72 latent frames (63,360 rows x 16 "
                                          "heads, 4 camera tokens each; numpy float64, %.1f s)" % dt}
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="c4", choices=sorted(workloads.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the c1-c3 attention rates reported beside the c4 line")
    ap.add_argument("--int8-attn", choices=("window", "cache"), default="window",
                    help="INT8 history: expand the window to bf16 once per layer-step (window) "
                         "or dequantise inside every attention workgroup (cache)")
    ap.add_argument("--counters-workload", action="store_true",
                    help="one calibration copy + one attention call, for rocprofv3 --pmc")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="FETCH_DIR WRITE_DIR [DRAM_DIR]: rocprofv3 --pmc outputs to summarise")
    ap.add_argument("--summarize-issue", metavar="DIR",
                    help="a rocprofv3 --pmc output over the issue counters to summarise")
    ap.add_argument("--issue-kernel", default=ATTN_KERNEL,
                    help="kernel whose dispatches --summarize-issue reads (with --train: dq_kernel, dkdv_kernel)")
    ap.add_argument("--camera", action="store_true",
                    help="the per-latent-frame camera cross-attention instead")
    ap.add_argument("--linear", action="store_true",
                    help="the INT8-weight linears of one block's video stream instead")
    ap.add_argument("--archive", action="store_true",
                    help="the CPU history archive instead: window fetch / segment store over PCIe, and "
                         "the fetch overlapped with an attention call")
    ap.add_argument("--train", action="store_true",
                    help="the packed training form instead: forward + backward of one layer's "
                         "attention over 13 packed segments (346,528 rows)")
    args = ap.parse_args()
    if args.summarize_counters:
        d = args.summarize_counters
        if len(d) not in (2, 3):
            ap.error("--summarize-counters takes FETCH_DIR WRITE_DIR [DRAM_DIR]")
        summarize_counters(args.config, d[0], d[1],
                           os.path.join(ROOT, "profiles", "attn_%s_counters.json" % args.config),
                           d[2] if len(d) == 3 else None)
        return
    if args.summarize_issue:
        if args.train:
            summarize_issue("train13", args.summarize_issue,
                            os.path.join(ROOT, "profiles", "%s_train13_issue.json" % args.issue_kernel),
                            kernel=args.issue_kernel,
                            workload_cmd="python3 bench.py --train --steps 1 --warmup 0 --no-cpu-baseline")
        else:
            summarize_issue(args.config, args.summarize_issue,
                            os.path.join(ROOT, "profiles", "attn_%s_issue.json" % args.config))
        return
    if args.counters_workload:
        counters_workload(args.config)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the attention would shard by heads; see the design notes).", file=sys.stderr)
        sys.exit(2)

    if args.train:
        train_bench(args)
        return
    if args.archive:
        archive_bench(args)
        return
    if args.linear:
        linear_bench(args)
        return
    if args.camera:
        camera_bench(args)
        return

    import torch
    import segment_causal_dit_amd as sc

    cfg = workloads.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g, h = cfg.tokens_per_frame, cfg.n_heads
    log("generating %s inputs" % cfg.name)
    inp = workloads.make_inputs(cfg)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q_pre, k_pre, v = bf(inp.q), bf(inp.k), bf(inp.v)
    q, k = q_pre.clone(), k_pre.clone()
    seg = cfg.segments[0]
    tl = seg.text_len
    n_vid = cfg.n_video
    pos = torch.from_numpy(inp.pos).to(dev)
    n_hist_frames = len(cfg.hist_t)
    cache = None
    if n_hist_frames:
        cache = sc.KVCache(cfg.n_slots, h, g, cfg.cache_dtype, dev)
        hk = bf(inp.hist_k)
        sc.rope3d_apply(hk, torch.from_numpy(inp.hist_pos).to(dev))
        sc.kv_cache_append(cache, 0, hk, bf(inp.hist_v))
        cache.slot_t[:] = inp.slot_t
        del hk
    expand = cache is not None and cfg.cache_dtype == "int8" and args.int8_attn == "window"
    win = sc.KVCache(min(cfg.window, n_hist_frames), h, g, "bf16", dev) if expand else None
    n_win = len(sc.window_select(cache.slot_t[:n_hist_frames], cfg.window)) if cache else 0
    ws = attn_workspace(sc, cfg.n_cur, h, [(0, tl, seg.text_valid)],
                        torch.zeros(n_win, dtype=torch.int32) if n_win else None,
                        win if expand else cache, dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = {k_: [] for k_ in ("rope", "dequant", "attn", "append")}

    def rec(name, fn):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        ev[name].append((a, b))

    def one_step():
        slots = sc.window_select(cache.slot_t[:n_hist_frames], cfg.window) if cache else None
        hist = torch.from_numpy(slots).to(dev, non_blocking=False) if cache else None
        acache, ahist = cache, hist
        if expand:
            acache, ahist = win, torch.arange(len(slots), dtype=torch.int32, device=dev)
        for _ in range(DENOISE_STEPS):
            rec("rope", lambda: (sc.rope3d_apply(q_pre[tl:], pos, x_out=q[tl:]),
                                 sc.rope3d_apply(k_pre[tl:], pos, x_out=k[tl:])))
            if expand:   # once per layer-step: a model's other layers reuse the buffer between steps
                rec("dequant", lambda: sc.kv_window_dequant(cache, hist, win))
            rec("attn", lambda: sc.segcausal_joint_attn(q, k, v, [(0, tl, seg.text_valid)],
                                                        cfg.sm_scale, cache=acache,
                                                        hist_slots=ahist, out=out, workspace=ws))
        if cache is not None and cfg.append:
            rec("append", lambda: sc.kv_cache_append(cache, n_hist_frames, k[tl:], v[tl:]))

    out = torch.empty_like(q)
    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    for k_ in ev:
        ev[k_].clear()
    log("timing %d steps" % args.steps)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        one_step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    def avg_ms(name):
        xs = [a.elapsed_time(b) for a, b in ev[name]]
        return float(np.mean(xs)) if xs else 0.0

    attn_ms, rope_ms, app_ms = avg_ms("attn"), avg_ms("rope"), avg_ms("append")
    deq_ms = avg_ms("dequant")
    deq_bytes = (cfg.n_hist_rows * h * (HEAD_DIM + 4 + HEAD_DIM * 2) * 2) if expand else 0
    flops = cfg.flops()
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    step_tflops = DENOISE_STEPS * flops / (ms_step * 1e-3) / 1e12
    vid_tok_s = DENOISE_STEPS * n_vid / (ms_step * 1e-3)
    rope_bytes = 2 * 2 * n_vid * h * HEAD_DIM * 2           # q and k, read + write
    app_bytes = n_vid * h * ((HEAD_DIM * 2 + HEAD_DIM + 4) * 2 if cfg.cache_dtype == "int8"
                             else HEAD_DIM * 2 * 2 * 2)
    log("attn %.3f ms (%.1f TFLOP/s, %.1f%% of bf16 peak)  rope q+k %.3f ms (%.0f GB/s)  "
        "append %.3f ms (%.0f GB/s)  step %.2f ms"
        % (attn_ms, attn_tflops, 100 * attn_tflops / PEAK_BF16_TFLOPS, rope_ms,
           rope_bytes / (rope_ms * 1e-3) / 1e9 if rope_ms else 0, app_ms,
           app_bytes / (app_ms * 1e-3) / 1e9 if app_ms else 0, ms_step))
    if expand:
        log("window dequant %.3f ms (%.0f GB/s)" % (deq_ms, deq_bytes / (deq_ms * 1e-3) / 1e9))
        # beside it: the same attention over the INT8 cache itself, the dequantisation fused into the
        # tile loads (bit-identical output); reported, not part of the step
        slots = sc.window_select(cache.slot_t[:n_hist_frames], cfg.window)
        hist = torch.from_numpy(slots).to(dev)
        fused = []
        for _ in range(4):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            sc.segcausal_joint_attn(q, k, v, [(0, tl, seg.text_valid)], cfg.sm_scale, cache=cache,
                                    hist_slots=hist, out=out, workspace=None)
            b.record(stream)
            fused.append((a, b))
        torch.cuda.synchronize()
        fused_ms = float(np.mean([a.elapsed_time(b) for a, b in fused[1:]]))
        fused_tflops = flops / (fused_ms * 1e-3) / 1e12
        log("attention over the INT8 cache (dequantisation in the tile loads) %.3f ms (%.1f TFLOP/s)"
            % (fused_ms, fused_tflops))

    traffic = measured_traffic(cfg, history_path(cfg, args.int8_attn))
    line = {
        "metric": METRIC,
        "value": round(step_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "%s: %d current queries (%d text + %d video) x %d heads x 128 over "
                        "%d %s history keys + the current segment; 8 denoising layer-steps "
                        "(RoPE q,k + %sattention) + window select + append per step"
                        % (cfg.name, cfg.n_cur, tl, n_vid, h, cfg.n_hist_rows, cfg.cache_dtype,
                           "INT8 window expanded to bf16 + " if expand else ""),
            "n_cur": cfg.n_cur, "n_hist_keys": cfg.n_hist_rows, "heads": h,
            "head_dim": HEAD_DIM, "cache": cfg.cache_dtype,
        },
        "video_tokens_per_s_per_layer_step": round(vid_tok_s, 1),
        "kernels_ms": {"attn": round(attn_ms, 4), "rope_qk": round(rope_ms, 4),
                       "append": round(app_ms, 4), "window_dequant": round(deq_ms, 4) if expand else None},
        "hbm_frac": {"rope_qk": round(rope_bytes / (rope_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
                     if rope_ms else None,
                     "append": round(app_bytes / (app_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
                     if app_ms else None,
                     "window_dequant": round(deq_bytes / (deq_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
                     if expand and deq_ms else None},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    if expand:
        line["int8_cache_attention"] = {"ms": round(fused_ms, 4), "tflops": round(fused_tflops, 3),
                                        "frac": round(fused_tflops / PEAK_BF16_TFLOPS, 4)}
    del q_pre, k_pre, q, k, v, out, cache, win
    torch.cuda.empty_cache()
    if args.config == "c4" and not args.no_other_configs:
        # the shorter configurations' attention, each against its own roofline
        line["other_configs"] = config_rates(["c1", "c2", "c3"])
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle sample)")
        line["cpu_baseline"] = cpu_baseline(cfg, inp)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
