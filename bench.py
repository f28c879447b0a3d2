#!/usr/bin/env python3
"""Benchmark of single-token decode attention over a KV cache on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--quick] [--no-cpu-baseline]

Prints ONE JSON line on stdout.  The headline `value` is the KV bytes the
Llama-3-8B-shaped GQA layer must read (B16, 32/8 heads, D128, 8192 tokens,
paged 16, bf16) divided by the wall time of one decode_attn_gqa call (split
kernel + log-sum-exp combine), K calls timed back to back with inputs resident
in HBM.  The other workloads (window + sinks, MLA, DSA, Quest page selection,
cache append) are reported under "workloads".  A step is one call of the hot
path on one batch.  Inputs rotate over copies so that the bytes a step reads
recur only after about 1 GiB of other reads: no step is served from the
256 MB Infinity Cache by a previous one.

Timing, per workload:
  * W warmup calls, then a clock ramp: calls keep running until `--ramp-ms`
    of wall time has passed (the GPU's clocks take tens of ms of sustained
    work to rise after the inputs were built on the CPU); reported as
    "ramp";
  * the step pass: K calls back to back between two synchronisations (the
    headline `ms_per_step` and `value`);
  * the kernel pass: the same K calls with the library's per-kernel timing,
    HIP events bound to the kernel dispatches on the launch stream
    (hipExtLaunchKernel), which exclude the launch gaps between kernels;
  * per-call statistics: each call bracketed by HIP events, median and
    p10/p90, once after an untimed 1 GiB scrub write before every call
    ("call_us", cold) and once with no scrub on one buffer ("warm_call_us",
    labelled warm).

`roofline` covers the dominant kernel (gqa_split): algorithmic bytes per
launch over its average duration from the kernel pass.  `read_ceiling` is
the best rate of a plain streaming-read probe over the same bytes.
`cpu_baseline` is the CPU oracle (plain fp64 C, OpenMP over rows) timed on
this host on the same workload; the same leg, the only one that uses the
oracle, also reports each configuration's error against it on sampled rows.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
ROTATE_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def copies_for(touched_bytes):
    """Copies to rotate over so that the bytes one step touches recur only
    after ~1 GiB of other reads (at most 8)."""
    return max(1, min(8, math.ceil(ROTATE_BYTES / max(1, touched_bytes))))


def pct(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 3), "p10": round(float(np.percentile(a, 10)), 3),
            "p90": round(float(np.percentile(a, 90)), 3)}


def sha256_of(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


# Kernels with committed rocprofv3 counter records (profiles/<name>_counters.json):
# name -> (bench --only workload, kernel-name pattern, source file, what one
# launch does).  The records are written by `bench.py --counter-summary DIR`
# from the counter passes listed in COUNTER_PASSES, each run as
#   rocprofv3 --pmc <counters> -d DIR/<workload>_<pass> -o run --output-format csv --
#       python3 bench.py --only <workload> --steps 20 --warmup 5 --ramp-ms 50
# and from the same FETCH_SIZE / WRITE_SIZE passes over `bench.py
# --calibrate-copy --steps 5` (DIR/copy_fetch, DIR/copy_write), which read and
# write exactly 1 GiB per launch and so give the counters' byte scale.
COUNTER_KERNELS = {
    "gqa_split": ("gqa", r"gqa_split_kernel", "gqa_decode.hip",
                  "GQA Llama-3-8B layer (B16, 32/8 heads, D128, 8192 tokens, paged 16, bf16): "
                  "K+V 536870912 bytes"),
    "mla_split": ("mla", r"mla_tile32_kernel<0(, (true|false))?>", "mla_decode.hip",
                  "MLA DeepSeek-V3 shape (B32, H128, 576-wide latent, 16384 tokens, bf16): "
                  "latent 603979776 bytes, 146028888064 flops"),
    "sparse_mla_split": ("dsa", r"mla_tile32_kernel<1(, (true|false))?>", "mla_decode.hip",
                         "sparse MLA over top-2048 of 65536 (B8, H128, bf16): "
                         "selected latent rows 18874368 bytes, 4563402752 flops"),
    "indexer_bf16": ("dsa", r"indexer_kernel<\d+, false>", "indexer.hip",
                     "DSA indexer (B8, 65536 tokens, 64 heads x 128, bf16 keys): "
                     "134217728 key bytes"),
    "indexer_fp8": ("dsa", r"indexer_kernel<\d+, true>", "indexer.hip",
                    "DSA indexer (B8, 65536 tokens, 64 heads x 128, fp8 e4m3 keys): "
                    "67108864 key bytes"),
}
COUNTER_PASSES = {
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
    "mfma": "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_LDS "
            "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE",
    "issue": "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_WAIT_INST_LDS "
             "SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VALU SQ_INSTS_SALU",
}


def counter_record(kernel):
    """The committed counter record of a kernel if it was taken on the current
    kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, "decode_attention_kv_flash_amd", "csrc", rec["source"])
    if rec.get("source_sha256") != sha256_of(src):
        return None
    return rec


def counter_traffic(kernel):
    """HBM bytes per launch from the committed counter record, or None."""
    rec = counter_record(kernel)
    return None if rec is None else rec["hbm_bytes_per_launch"]


def counter_fields(kernel):
    """Counter-measured fields for a workload record (None when stale)."""
    rec = counter_record(kernel)
    if rec is None:
        return {"counters": None}
    return {"counters": {k: rec[k] for k in ("hbm_bytes_per_launch", "fetch_bytes_per_launch",
                                              "write_bytes_per_launch", "mfma_busy_frac",
                                              "lds_bank_conflict_per_lds_inst")}}


def _pmc_means(csv_path, pattern):
    """Per-counter mean over the dispatches of kernels matching pattern (a
    counter's per-dispatch value is the sum of its rows)."""
    import csv
    import re
    per = {}
    rx = re.compile(pattern)
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if not rx.search(r["Kernel_Name"]):
                continue
            d = per.setdefault(r["Counter_Name"], {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return {c: (sum(v.values()) / len(v), len(v)) for c, v in per.items()}


def counter_summary(pmc_dir):
    """Writes profiles/<kernel>_counters.json and a text summary per kernel
    from the counter passes under pmc_dir."""
    import glob
    def csv_of(tag):
        return glob.glob(os.path.join(pmc_dir, tag, "*counter_collection.csv"))[0]
    copy_fetch = _pmc_means(csv_of("copy_fetch"), r"copyBuffer|copy_kernel|direct_copy")["FETCH_SIZE"][0]
    copy_write = _pmc_means(csv_of("copy_write"), r"copyBuffer|copy_kernel|direct_copy")["WRITE_SIZE"][0]
    fetch_scale = (1 << 30) / (copy_fetch * 1024)
    write_scale = (1 << 30) / (copy_write * 1024)
    cmd = ("cd /tmp && rocprofv3 --pmc {ctr} -d <out>/{tag} -o run --output-format csv -- "
           "python3 <repo>/bench.py {args}")
    wl_args = "--only {w} --steps 20 --warmup 5 --ramp-ms 50"
    for name, (w, pattern, source, what) in COUNTER_KERNELS.items():
        vals = {}
        for p in COUNTER_PASSES:
            try:
                vals.update(_pmc_means(csv_of(f"{w}_{p}"), pattern))
            except IndexError:
                pass
        if "FETCH_SIZE" not in vals:
            log(f"[counters] no passes for {name}")
            continue
        v = {c: x for c, (x, _) in vals.items()}
        n_disp = vals["FETCH_SIZE"][1]
        fetch_b = v["FETCH_SIZE"] * 1024 * fetch_scale
        write_b = v["WRITE_SIZE"] * 1024 * write_scale
        rec = {
            "kernel": name, "kernel_pattern": pattern, "workload": what,
            "source": source,
            "source_sha256": sha256_of(os.path.join(ROOT, "decode_attention_kv_flash_amd", "csrc", source)),
            "dispatches": n_disp,
            "fetch_kib_per_dispatch": round(v["FETCH_SIZE"], 1),
            "write_kib_per_dispatch": round(v["WRITE_SIZE"], 1),
            "copy_1GiB_fetch_kib": round(copy_fetch, 1), "copy_1GiB_write_kib": round(copy_write, 1),
            "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
            "fetch_bytes_per_launch": int(fetch_b), "write_bytes_per_launch": int(write_b),
            "hbm_bytes_per_launch": int(fetch_b + write_b),
            # MFMA pipes busy over all SIMDs (4 per CU) of the CUs the kernel occupied
            "mfma_busy_frac": round(v["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * v["SQ_BUSY_CU_CYCLES"]), 4)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in v else None,
            "lds_bank_conflict_per_lds_inst": round(v["SQ_LDS_BANK_CONFLICT"] / max(v["SQ_INSTS_LDS"], 1), 4)
            if "SQ_LDS_BANK_CONFLICT" in v else None,
            "wave_cycle_fracs": {k: round(v[k] / v["SQ_WAVE_CYCLES"], 4)
                                 for k in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
                                           "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VALU")
                                 if k in v and "SQ_WAVE_CYCLES" in v},
            "counters_per_dispatch": {k: round(x, 1) for k, x in sorted(v.items())},
            "commands": {p: cmd.format(ctr=ctr, tag=f"{w}_{p}", args=wl_args.format(w=w))
                         for p, ctr in COUNTER_PASSES.items()},
        }
        rec["commands"]["copy_fetch"] = cmd.format(ctr="FETCH_SIZE", tag="copy_fetch",
                                                   args="--calibrate-copy --steps 5")
        rec["commands"]["copy_write"] = cmd.format(ctr="WRITE_SIZE", tag="copy_write",
                                                   args="--calibrate-copy --steps 5")
        with open(os.path.join(ROOT, "profiles", f"{name}_counters.json"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        lines = [f"# {name} counters: {what}", "",
                 "rocprofv3 --pmc, one counter set per run (passes below); values are means over the",
                 f"{n_disp} dispatches of kernels matching /{pattern}/.  FETCH_SIZE and WRITE_SIZE are",
                 "scaled by the same counters on a plain 1 GiB device copy (bench.py --calibrate-copy).", ""]
        for p, c in rec["commands"].items():
            lines.append(f"{p}: {c}")
        lines += ["",
                  f"FETCH_SIZE  {v['FETCH_SIZE']:14.1f} KiB/dispatch x {fetch_scale:.4f} = {int(fetch_b):13d} bytes",
                  f"WRITE_SIZE  {v['WRITE_SIZE']:14.1f} KiB/dispatch x {write_scale:.4f} = {int(write_b):13d} bytes",
                  f"HBM bytes per launch {int(fetch_b + write_b)}"]
        if rec["mfma_busy_frac"] is not None:
            lines.append(f"MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES)) {rec['mfma_busy_frac']:.4f}")
        if rec["lds_bank_conflict_per_lds_inst"] is not None:
            lines.append(f"LDS bank conflict cycles per LDS instruction {rec['lds_bank_conflict_per_lds_inst']:.4f}")
        for k, x in rec["wave_cycle_fracs"].items():
            lines.append(f"{k} / SQ_WAVE_CYCLES {x:.4f}")
        lines += ["", "counters per dispatch:"]
        lines += [f"  {k:28s} {x:16.1f}" for k, x in sorted(v.items())]
        lines.append(f"\nkernel source {source} sha256 {rec['source_sha256']}")
        with open(os.path.join(ROOT, "profiles", f"{name}_counters.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
        log(f"[counters] {name}: {int(fetch_b + write_b)} HBM bytes/launch, mfma busy {rec['mfma_busy_frac']}")


# Algorithmic work per launch of the dominant kernels, for the kernel-trace
# summaries: kernel-name pattern -> (bytes, flops or None).
TRACE_WORK = {
    "gqa": {r"gqa_split_kernel": (536870912, None)},
    "swa": {},
    "layouts": {r"gqa_split_kernel": (536870912, None)},
    "mla": {r"mla_tile32_kernel<0(, (true|false))?>": (603979776, 146028888064)},
    "dsa": {r"indexer_kernel<\d+, false>": (134217728, None),
            r"indexer_kernel<\d+, true>": (67108864, None),
            r"mla_tile32_kernel<1(, (true|false))?>": (18874368, 4563402752)},
    "quest": {},
    "append": {},
}


def _short_name(name):
    import re
    n = re.sub(r"^void ", "", name)
    n = re.sub(r"dattn::\(anonymous namespace\)::", "", n)
    return re.sub(r"\((dattn::)?\w+Args\)$", "", n)


def trace_summary(trace_dir, workload, steps, out_name, title):
    """profiles/<out_name>.txt from a rocprofv3 --kernel-trace --stats run of
    `bench.py --only <workload> --steps <steps>`: per kernel and grid, the
    durations of the step and kernel passes (the 2 x steps dispatches before
    the two per-call passes), which follow the warmup and the clock ramp."""
    import csv
    import glob
    import re
    path = glob.glob(os.path.join(trace_dir, "*kernel_trace.csv"))[0]
    if workload == "quick":  # the headline workload as the full benchmark runs it
        bench_args = f"--quick --steps {steps} --warmup 20 --no-cpu-baseline"
        workload = "gqa"
    else:
        bench_args = f"--only {workload} --steps {steps} --warmup 20"
    groups = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if "dattn::" not in r["Kernel_Name"]:
                continue
            key = (r["Kernel_Name"], (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"])))
            g = groups.setdefault(key, {"d": [], "row": r})
            g["d"].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    K = steps
    lines = [f"# {title}", "",
             "rocprofv3 kernel trace (--kernel-trace --stats) of one benchmark workload; per kernel",
             f"and grid, durations over its step and kernel passes ({K} calls each, back to back,",
             "after the warmup and the clock ramp; the per-call passes that follow are left out).",
             f"command: cd /tmp && rocprofv3 --kernel-trace --stats -d <out> -o run --output-format csv -- "
             f"python3 <repo>/bench.py {bench_args}", "",
             f"{'kernel':52s} {'grid (threads)':>20s} {'wg':>5s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} "
             f"{'max us':>9s} {'vgpr':>5s} {'agpr':>5s} {'lds':>7s} {'scratch':>7s}"]
    for (name, grid), g in sorted(groups.items(), key=lambda kv: kv[1]["d"][0][0]):
        d = [x for _, x in sorted(g["d"])]
        n = len(d)
        # the tail of each group's dispatches is [step, kernel, cold, warm] x K
        win = d[n - 4 * K: n - 2 * K] if n >= 4 * K else d
        us = [x / 1e3 for x in win]
        r = g["row"]
        sn = _short_name(name)
        lines.append(f"{sn[:52]:52s} {str(grid):>20s} {r['Workgroup_Size_X']:>5s} {len(us):6d} "
                     f"{sum(us) / len(us):9.2f} {min(us):9.2f} {max(us):9.2f} {r['VGPR_Count']:>5s} "
                     f"{r['Accum_VGPR_Count']:>5s} {r['LDS_Block_Size']:>7s} {r['Scratch_Size']:>7s}")
        for pat, (nb, nf) in TRACE_WORK.get(workload, {}).items():
            if re.search(pat, name):
                avg = sum(us) / len(us)
                lines.append(f"    algorithmic bytes {nb} -> {gbs(nb, avg):.1f} GB/s "
                             f"({100 * gbs(nb, avg) / HBM_PEAK_GBS:.1f}% of 8 TB/s)")
                if nf:
                    lines.append(f"    algorithmic flops {nf} -> {tflops(nf, avg):.1f} TFLOP/s "
                                 f"({100 * tflops(nf, avg) / BF16_PEAK_TFLOPS:.1f}% of 2.5 PFLOP/s bf16)")
    with open(os.path.join(ROOT, "profiles", out_name + ".txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"[trace] wrote profiles/{out_name}.txt")


class Timer:
    def __init__(self, api, torch, ramp_ms):
        self.api, self.torch, self.ramp_ms = api, torch, ramp_ms
        # written before each cold per-call sample: evicts the 256 MB
        # Infinity Cache and the L2s
        self.scrub = torch.empty(ROTATE_BYTES, dtype=torch.uint8, device="cuda:0")

    def ramp(self, step, start):
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n = 0
        while (time.perf_counter() - t0) * 1e3 < self.ramp_ms:
            for _ in range(16):
                step(start + n)
                n += 1
            torch.cuda.synchronize()
        return {"calls": n, "ms": round((time.perf_counter() - t0) * 1e3, 1)}

    def per_call(self, step, steps, scrub):
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i, (a, b) in enumerate(ev):
            if scrub:
                self.scrub.fill_(i & 255)
            a.record()
            step(i if scrub else 0)
            b.record()
        torch.cuda.synchronize()
        return pct([1e3 * a.elapsed_time(b) for a, b in ev])

    def run(self, step, steps, warmup, kernels):
        """Warmup, clock ramp, then the step pass (wall time), the kernel pass
        (dispatch-bound per-kernel events) and the per-call passes."""
        torch, api = self.torch, self.api
        for i in range(warmup):
            step(i)
        ramp = self.ramp(step, warmup)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        api.profile_reset()
        api.profile_enable(True)
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        api.profile_enable(False)
        per_kernel = {}
        for k in kernels:
            tot, cnt = api.profile_read(k)
            per_kernel[k] = {"avg_us": 1e3 * tot / cnt if cnt else None, "launches": cnt}
        api.profile_reset()
        cold = self.per_call(step, steps, scrub=True)
        warm = self.per_call(step, steps, scrub=False)
        return {"wall_ms": 1e3 * (t1 - t0) / steps, "event_ms": e0.elapsed_time(e1) / steps,
                "kernels": per_kernel, "call_us": cold, "warm_call_us": warm, "ramp": ramp}


def stats(r):
    """The timing fields every workload record carries."""
    return {"call_us": r["call_us"], "warm_call_us": r["warm_call_us"], "ramp": r["ramp"]}


def check(lib, rc):
    if rc != 0:
        raise RuntimeError(lib.dattn_last_error().decode())


def bench_gqa(x, timer, steps, warmup, torch, lib, sink_logits=None):
    """decode_attn_gqa on a (paged) GQA workload (decode_attn_gqa_sink when
    sink_logits, fp32 [Hq], is given); returns the timing record."""
    dev = torch.device("cuda:0")
    q, sl = x.q.to(dev), x.seq_lens.to(dev)
    pt = x.page_table.to(dev) if x.page_table is not None else None
    R = copies_for(x.kv_bytes())
    kc = [x.k_cache.to(dev) for _ in range(R)]
    vc = [x.v_cache.to(dev) for _ in range(R)]
    out = torch.empty_like(q)
    lse = torch.empty(x.B, x.Hq, dtype=torch.float32, device=dev)
    max_pages = x.max_pages
    nbytes = lib.decode_attn_gqa_workspace(x.B, x.Hq, x.Hkv, x.D, x.page_size, max_pages,
                                           x.window, x.n_sink, 0)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    dt = 1 if x.q.dtype == torch.bfloat16 else 0
    if sink_logits is None:
        args = [(ptr(q), ptr(kc[r]), ptr(vc[r]), ptr(sl), ptr(pt), x.window, x.n_sink, ptr(out),
                 ptr(lse), x.B, x.Hq, x.Hkv, x.D, x.page_size, max_pages, dt,
                 ctypes.c_float(x.scale), 0, ptr(ws), nbytes, stream) for r in range(R)]
        fn = lib.decode_attn_gqa
    else:
        sk = sink_logits.to(dev)
        args = [(ptr(q), ptr(kc[r]), ptr(vc[r]), ptr(sl), ptr(pt), x.window, x.n_sink, ptr(sk),
                 ptr(out), ptr(lse), x.B, x.Hq, x.Hkv, x.D, x.page_size, max_pages, dt,
                 ctypes.c_float(x.scale), 0, ptr(ws), nbytes, stream) for r in range(R)]
        fn = lib.decode_attn_gqa_sink

    def step(i):
        check(lib, fn(*args[i % R]))

    rec = timer.run(step, steps, warmup, ["gqa_split", "lse_combine"])
    rec["copies"] = R
    rec["out"], rec["lse"] = out, lse
    return rec


def bench_mla(m, timer, steps, warmup, torch, lib):
    dev = torch.device("cuda:0")
    q, sl = m.q.to(dev), m.seq_lens.to(dev)
    R = copies_for(m.kv_bytes())
    lat = [m.latent.to(dev) for _ in range(R)]
    out = torch.empty(m.B, m.H, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(m.B, m.H, dtype=torch.float32, device=dev)
    nbytes = lib.decode_attn_mla_workspace(m.B, m.H, 512, m.S_max, 0)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [(ptr(q), ptr(lat[r]), ptr(sl), None, ptr(out), ptr(lse), m.B, m.H, 512, 64, m.S_max,
             m.S_max, 1, 1, ctypes.c_float(m.scale), 0, ptr(ws), nbytes, stream) for r in range(R)]
    fn = lib.decode_attn_mla

    def step(i):
        check(lib, fn(*args[i % R]))

    rec = timer.run(step, steps, warmup, ["mla_split", "lse_combine"])
    rec["copies"] = R
    rec["out"], rec["lse"] = out, lse
    return rec


def bench_dsa(d, timer, steps, warmup, torch, lib):
    """Indexer + top-k over the full context, then sparse MLA over the selection."""
    dev = torch.device("cuda:0")
    m = d.mla
    B, Hi, Di = d.q_i.shape
    S = d.k_i.shape[1]
    # each step reads every key of the indexer cache and the selected latent
    # rows; both rotate over R copies (the latent's selected rows are 18.9 MB
    # a step, so a copy is read again only after R - 1 indexer passes)
    R = copies_for(d.indexer_bytes())
    qi, w, sl = d.q_i.to(dev), d.w.to(dev), d.seq_lens.to(dev)
    ki = [d.k_i.to(dev) for _ in range(R)]
    q = m.q.to(dev)
    lat = [m.latent.to(dev) for _ in range(R)]
    idx = torch.empty(B, d.topk, dtype=torch.int32, device=dev)
    scores = torch.empty(B, S, dtype=torch.float32, device=dev)
    out = torch.empty(B, m.H, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, m.H, dtype=torch.float32, device=dev)
    nbytes = lib.sparse_mla_attn_workspace(B, m.H, 512, d.topk, 0)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    ibytes = lib.dsa_indexer_topk_workspace(B, S, d.topk)
    iws = torch.empty(max(ibytes, 1), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    a1 = [(ptr(qi), ptr(w), ptr(ki[r]), ptr(sl), d.topk, ptr(idx), ptr(scores), B, Hi, Di, S, 1,
           ptr(iws), ibytes, stream) for r in range(R)]
    a2 = [(ptr(q), ptr(lat[r]), ptr(idx), d.topk, ptr(out), ptr(lse), B, m.H, 512, 64, m.S_max, 1,
           ctypes.c_float(m.scale), 0, ptr(ws), nbytes, stream) for r in range(R)]

    def step(i):
        check(lib, lib.dsa_indexer_topk(*a1[i % R]))
        check(lib, lib.sparse_mla_attn(*a2[i % R]))

    rec = timer.run(step, steps, warmup, ["indexer_scores", "topk_select", "sparse_mla_split",
                                          "lse_combine"])
    rec["copies"] = R
    rec["out"], rec["lse"], rec["idx"] = out, lse, idx.clone()
    # the indexer with its inputs in fp8 e4m3 (exact for these integers): half the key bytes
    qi8 = qi.to(torch.float8_e4m3fn)
    ki8 = [t.to(torch.float8_e4m3fn) for t in ki]
    a8 = [(ptr(qi8), ptr(w), ptr(ki8[r]), ptr(sl), d.topk, ptr(idx), ptr(scores), B, Hi, Di, S, 2,
           ptr(iws), ibytes, stream) for r in range(R)]
    r8 = timer.run(lambda i: check(lib, lib.dsa_indexer_topk(*a8[i % R])), steps, warmup,
                   ["indexer_scores", "topk_select"])
    rec["fp8"] = r8
    return rec


def bench_quest(x, timer, steps, warmup, torch, lib, budget):
    """Quest on a GQA workload: per query head the `budget` 16-token blocks with
    the largest key bounds plus the partial block (bounds, top-k, attention
    over the chosen blocks, combine), and the block-summary build."""
    dev = torch.device("cuda:0")
    q, sl, pt = x.q.to(dev), x.seq_lens.to(dev), x.page_table.to(dev)
    # a step reads the block summaries (1/16 of K) and the chosen blocks' K/V
    # (about 60% of the layer for these inputs)
    R = copies_for(x.kv_bytes() // 2)
    kc = [x.k_cache.to(dev) for _ in range(R)]
    vc = [x.v_cache.to(dev) for _ in range(R)]
    max_pages = x.page_table.shape[1]
    nblk = x.page_size * max_pages // 16
    kmm = [torch.empty(x.B, x.Hkv, nblk, 2, x.D, dtype=x.k.dtype, device=dev) for _ in range(R)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    dt = 1 if x.q.dtype == torch.bfloat16 else 0
    mm = [(ptr(kc[r]), ptr(sl), ptr(pt), ptr(kmm[r]), 0, x.B, x.Hkv, x.D, x.page_size, max_pages, dt,
           stream) for r in range(R)]
    for a in mm:
        check(lib, lib.quest_page_minmax(*a))
    out = torch.empty_like(q)
    lse = torch.empty(x.B, x.Hq, dtype=torch.float32, device=dev)
    nbytes = lib.decode_attn_quest_workspace(x.B, x.Hq, x.Hkv, x.D, x.page_size, max_pages, budget, dt, 0)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    args = [(ptr(q), ptr(kc[r]), ptr(vc[r]), ptr(kmm[r]), ptr(sl), ptr(pt), budget, ptr(out), ptr(lse),
             None, x.B, x.Hq, x.Hkv, x.D, x.page_size, max_pages, dt, ctypes.c_float(x.scale), 0,
             ptr(ws), nbytes, stream) for r in range(R)]
    rec = timer.run(lambda i: check(lib, lib.decode_attn_quest(*args[i % R])), steps, warmup,
                    ["quest_bounds", "topk_select", "quest_union", "gqa_split", "lse_combine"])
    # the chosen blocks, for the bytes the attention reads once per KV head
    sel = torch.empty(x.B, x.Hq, budget, dtype=torch.int32, device=dev)
    a0 = list(args[0])
    a0[9] = ptr(sel)
    check(lib, lib.decode_attn_quest(*a0))
    torch.cuda.synchronize()
    rec["selected"] = sel.cpu()
    # the summary of every block, and the refresh of one block per sequence
    rec["minmax_full"] = timer.run(lambda i: check(lib, lib.quest_page_minmax(*mm[i % R])), steps,
                                   warmup // 4, ["quest_minmax"])
    last = int(x.seq_lens.min()) // 16 - 1
    inc = [a[:4] + (last,) + a[5:] for a in mm]
    rec["minmax_one_block"] = timer.run(lambda i: check(lib, lib.quest_page_minmax(*inc[i % R])), steps,
                                        warmup // 4, ["quest_minmax"])
    rec["copies"] = R
    return rec


def quest_bytes(x, budget, selected=None):
    """Algorithmic bytes of one Quest step: block summaries, the bounds
    written and read back by the select, and K/V of the chosen tokens: per
    query head, and (given the chosen blocks [B, Hq, budget]) once per KV head
    for the union of its query heads' blocks."""
    import torch
    esz = x.k.element_size()
    G = x.Hq // x.Hkv
    row = 2 * x.D * esz  # K + V bytes of one token of one KV head
    summ = per_head = bounds = union = 0
    for b, L in enumerate(x.seq_lens.tolist()):
        nf = L // 16
        summ += x.Hkv * nf * 2 * x.D * esz
        bounds += 2 * x.Hq * nf * 4
        per_head += x.Hq * (min(budget, nf) * 16 + L % 16) * row
        if selected is not None:
            for g in range(x.Hkv):
                s = selected[b, g * G:(g + 1) * G]
                n = torch.unique(s[s >= 0]).numel()
                union += (n * 16 + L % 16) * row
    return summ, bounds, per_head, union


def bench_append(timer, steps, warmup, torch, lib):
    """Cache append of one decode step: K/V rows of the Llama-3-8B-shaped GQA
    layer (B16, 8 KV heads, D128, paged 16), MLA latent rows (B32 x 576) and
    indexer keys (B8 x 128).  Each moves its rows once from the new-row
    buffer into the cache (bytes = 2 x rows)."""
    dev = torch.device("cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    g = torch.Generator().manual_seed(7)
    res = {}
    # GQA: 8192 tokens per sequence in a randomly permuted paged cache
    B, Hkv, D, P, L = 16, 8, 128, 16, 8192
    pages = B * L // P
    kc = torch.empty(pages, Hkv, P, D, dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    pt = torch.randperm(pages, generator=g).view(B, L // P).to(torch.int32).to(dev)
    kn = torch.randn(B, Hkv, D, generator=g).to(torch.bfloat16).to(dev)
    vn = torch.randn(B, Hkv, D, generator=g).to(torch.bfloat16).to(dev)
    pos = torch.full((B,), L - 1, dtype=torch.int32, device=dev)
    a = (ptr(kn), ptr(vn), ptr(kc), ptr(vc), ptr(pos), ptr(pt), B, Hkv, D, P, L // P, 0, 0, 1, stream)
    r = timer.run(lambda i: check(lib, lib.kv_append_gqa(*a)), steps, warmup, ["kv_append"])
    nb = 2 * 2 * B * Hkv * D * 2
    res["gqa_b16_kv8_d128_paged16"] = {"us": round(r["kernels"]["kv_append"]["avg_us"], 2),
                                       "bytes": nb, "GB/s": round(gbs(nb, r["kernels"]["kv_append"]["avg_us"]), 1)}
    del kc, vc
    for name, Bx, row, S in (("latent_b32_576", 32, 576, 16384), ("indexer_b8_128", 8, 128, 65536)):
        cache = torch.empty(Bx, S, row, dtype=torch.bfloat16, device=dev)
        new = torch.randn(Bx, row, generator=g).to(torch.bfloat16).to(dev)
        p2 = torch.full((Bx,), S - 1, dtype=torch.int32, device=dev)
        a2 = (ptr(new), ptr(cache), ptr(p2), None, Bx, row, S, 1, 1, stream)
        r = timer.run(lambda i: check(lib, lib.kv_append_rows(*a2)), steps, warmup, ["kv_append"])
        nb = 2 * Bx * row * 2
        res[name] = {"us": round(r["kernels"]["kv_append"]["avg_us"], 2), "bytes": nb,
                     "GB/s": round(gbs(nb, r["kernels"]["kv_append"]["avg_us"]), 1)}
        del cache
    return res


def gbs(nbytes, us):
    return None if not us else nbytes / (us * 1e-6) / 1e9


def tflops(flops, us):
    return None if not us else flops / (us * 1e-6) / 1e12


def rows_sample(n_rows, k, seed):
    """Deterministic sample of k flat row ids, the first and last included."""
    import torch
    g = torch.Generator().manual_seed(seed)
    pick = torch.randperm(n_rows, generator=g)[: max(0, k - 2)].tolist()
    return sorted(set([0, n_rows - 1] + pick))


def err_record(got, want, tol):
    """Max per-row ||x - y||_inf / ||y||_inf and the normwise ||x - y||_2 / ||y||_2."""
    import oracle
    import torch
    got = torch.as_tensor(got, dtype=torch.float64)
    want = torch.as_tensor(want, dtype=torch.float64)
    nw = float((got - want).norm() / want.norm()) if want.norm() > 0 else float((got - want).norm())
    return {"max_row_rel_err": float(f"{oracle.rel_err_rows(got, want):.3e}"),
            "normwise_rel_err": float(f"{nw:.3e}"), "rows": int(got.shape[0]), "tol": tol}


def gqa_error(x, rec, n_rows=48, seed=0):
    """The cpu_baseline leg: a GQA workload's output on sampled rows against the oracle."""
    import oracle
    rows = rows_sample(x.B * x.Hq, n_rows, seed)
    want, _ = oracle.gqa(x.q, x.k, x.v, x.seq_lens, window=x.window, n_sink=x.n_sink, scale=x.scale,
                         rows=rows)
    got = rec["out"].float().cpu().reshape(-1, x.D)[rows]
    return err_record(got, want, 1e-5 if x.q.dtype.itemsize == 4 else 2e-2)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--ramp-ms", type=float, default=200.0,
                    help="wall time of calls before each timed region (clock ramp)")
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--only", choices=["gqa", "swa", "layouts", "mla", "dsa", "append", "quest", "read"],
                    help="time one workload and print its record (for profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="time a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counter-summary", metavar="DIR",
                    help="write profiles/<kernel>_counters.{json,txt} from rocprofv3 counter passes in DIR")
    ap.add_argument("--trace-summary", nargs=4, metavar=("DIR", "WORKLOAD", "NAME", "TITLE"),
                    help="write profiles/NAME.txt from a rocprofv3 kernel trace in DIR of "
                         "bench.py --only WORKLOAD --steps STEPS")
    args = ap.parse_args()
    if args.trace_summary:
        d, w, name, title = args.trace_summary
        trace_summary(d, w, args.steps, name, title)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not "
              "supported: the decode-attention kernels run on a single GPU and this build has "
              "no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_attention_kv_flash_amd import api
    from decode_attention_kv_flash_amd import workloads as wl
    lib = api.lib()
    torch.cuda.set_device(0)
    steps, warmup = args.steps, args.warmup
    if args.calibrate_copy:
        calibrate_copy(torch, steps)
        return
    timer = Timer(api, torch, args.ramp_ms)
    if args.only:
        only(args.only, timer, steps, warmup, torch, lib, wl)
        return
    cpu = not args.no_cpu_baseline
    errors = {}

    # ---- headline: Llama-3-8B-shaped GQA layer --------------------------------
    log("[bench] generating gqa config (B16, 32/8 heads, D128, 8192 tokens, paged 16, bf16)")
    x2 = wl.config2_llama3_8b_gqa()
    bytes2 = x2.kv_bytes()
    flops2 = x2.attended_tokens() * 4 * x2.Hq * x2.D  # 4 S n_h d_h per sequence
    r2 = bench_gqa(x2, timer, steps, warmup, torch, lib)
    split_us = r2["kernels"]["gqa_split"]["avg_us"]
    log(f"[bench] gqa: {r2['wall_ms']*1e3:.1f} us/step wall, split kernel {split_us:.1f} us")
    if cpu:
        errors["config2_" + x2.name] = gqa_error(x2, r2, seed=2)
    value = bytes2 / (r2["wall_ms"] * 1e-3) / 1e9
    achieved = gbs(bytes2, split_us)
    log("[bench] streaming-read ceiling")
    ceiling = read_ceiling(timer, torch, lib, bytes2, steps)
    result = {
        "metric": "decode-attention KV GB/s read (% of MI355X HBM peak); MLA/DSA TFLOP/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(r2["wall_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": x2.name,
            "batch": x2.B, "q_heads": x2.Hq, "kv_heads": x2.Hkv, "head_dim": x2.D,
            "context": int(x2.seq_lens[0]), "page_size": x2.page_size,
            "kv_bytes_per_step": bytes2, "cache_copies_rotated": r2["copies"],
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "pct_of_read_ceiling": round(100 * value / ceiling["GB/s"], 2),
        },
        "roofline": {
            "kernel": "gqa_split",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": counter_traffic("gqa_split"),
            "algorithmic_bytes_per_launch": bytes2,
            "avg_launch_us": round(split_us, 2),
            "frac_of_read_ceiling": round(achieved / ceiling["GB/s"], 4),
        },
        "read_ceiling": ceiling,
        "clock_ramp_ms": args.ramp_ms,
        "workloads": {
            "gqa_llama3_8b": {"step_us": round(r2["wall_ms"] * 1e3, 2), "GB/s": round(value, 1),
                              "split_kernel": counter_fields("gqa_split"),
                              "TFLOP/s": round(flops2 / (r2["wall_ms"] * 1e-3) / 1e12, 3),
                              "kernels_us": {k: v["avg_us"] for k, v in r2["kernels"].items()},
                              **stats(r2)},
        },
    }
    del r2
    if not args.quick:
        budget = 128  # blocks of 16: 2048 tokens per query head
        log(f"[bench] quest on the gqa config, budget {budget} blocks")
        rq = bench_quest(x2, timer, steps, warmup, torch, lib, budget)
        kq = rq["kernels"]
        summ, bnd, selb, unib = quest_bytes(x2, budget, rq.pop("selected"))
        kbytes = x2.k.element_size() * x2.Hkv * x2.D * int(x2.seq_lens.sum())
        mm_us = rq["minmax_full"]["kernels"]["quest_minmax"]["avg_us"]
        result["workloads"]["quest_llama3_8b_budget2048"] = {
            "step_us": round(rq["wall_ms"] * 1e3, 2),
            "dense_step_us": result["workloads"]["gqa_llama3_8b"]["step_us"],
            "bytes_per_step": summ + bnd + unib,
            "GB/s": round((summ + bnd + unib) / (rq["wall_ms"] * 1e-3) / 1e9, 1),
            "kv_bytes_per_head_sum": selb,
            "kv_bytes_union_per_kv_head": unib,
            "bounds_GB/s": round(gbs(summ, kq["quest_bounds"]["avg_us"]), 1),
            "attention_GB/s": round(gbs(unib, kq["gqa_split"]["avg_us"]), 1),
            "topk_us": kq["topk_select"]["avg_us"],
            "kernels_us": {k: v["avg_us"] for k, v in kq.items()},
            "copies": rq["copies"],
            "minmax_all_blocks_us": round(mm_us, 2),
            "minmax_all_blocks_GB/s": round(gbs(kbytes, mm_us), 1),
            "minmax_one_block_us": round(rq["minmax_one_block"]["kernels"]["quest_minmax"]["avg_us"], 2),
            **stats(rq)}
        del rq
    del x2
    torch.cuda.empty_cache()

    if not args.quick:
        log("[bench] generating window+sinks config (B32, lens U[4096,32768], W4096 + 4 sinks)")
        x3 = wl.config3_swa_sinks()
        b3 = x3.kv_bytes()
        r3 = bench_gqa(x3, timer, steps, warmup, torch, lib)
        if cpu:
            errors["config3_" + x3.name] = gqa_error(x3, r3, seed=3)
        result["workloads"]["swa4096_sinks4"] = {
            "step_us": round(r3["wall_ms"] * 1e3, 2),
            "GB/s": round(b3 / (r3["wall_ms"] * 1e-3) / 1e9, 1),
            "split_kernel_GB/s": round(gbs(b3, r3["kernels"]["gqa_split"]["avg_us"]), 1),
            "kv_bytes_per_step": b3, "copies": r3["copies"],
            "kernels_us": {k: v["avg_us"] for k, v in r3["kernels"].items()}, **stats(r3)}
        del r3
        # the same workload with an explicit sink logit per head
        sk = torch.linspace(-2.0, 2.0, x3.Hq, dtype=torch.float32)
        r3s = bench_gqa(x3, timer, steps, warmup, torch, lib, sink_logits=sk)
        result["workloads"]["swa4096_sinks4_sink_logits"] = {
            "step_us": round(r3s["wall_ms"] * 1e3, 2),
            "GB/s": round(b3 / (r3s["wall_ms"] * 1e-3) / 1e9, 1),
            "split_kernel_GB/s": round(gbs(b3, r3s["kernels"]["gqa_split"]["avg_us"]), 1),
            "kv_bytes_per_step": b3,
            "kernels_us": {k: v["avg_us"] for k, v in r3s["kernels"].items()}, **stats(r3s)}
        del x3, r3s
        torch.cuda.empty_cache()

        result["workloads"]["gqa_head_layouts"] = bench_layouts(timer, steps, warmup, torch, lib, wl)

        log("[bench] generating MLA config (B32, H128, latent 576, 16384 tokens)")
        m4 = wl.config4_mla()
        r4 = bench_mla(m4, timer, steps, warmup, torch, lib)
        b4, f4 = m4.kv_bytes(), m4.flops()
        us4 = r4["kernels"]["mla_split"]["avg_us"]
        if cpu:
            import oracle
            rows = rows_sample(m4.B * m4.H, 48, 4)
            want, _ = oracle.mla(m4.q, m4.latent, m4.seq_lens, scale=m4.scale, rows=rows)
            errors["config4_" + m4.name] = err_record(r4["out"].float().cpu().reshape(-1, 512)[rows], want, 2e-2)
        result["workloads"]["mla_dsv3"] = {
            "step_us": round(r4["wall_ms"] * 1e3, 2),
            "TFLOP/s": round(f4 / (r4["wall_ms"] * 1e-3) / 1e12, 1),
            "GB/s": round(b4 / (r4["wall_ms"] * 1e-3) / 1e9, 1),
            "split_kernel_TFLOP/s": round(tflops(f4, us4), 1),
            "mfma_frac_of_bf16_peak": round(tflops(f4, us4) / BF16_PEAK_TFLOPS, 4),
            "split_kernel_hbm_frac": round(gbs(b4, us4) / HBM_PEAK_GBS, 4),
            "split_kernel": counter_fields("mla_split"),
            "copies": r4["copies"],
            "kernels_us": {k: v["avg_us"] for k, v in r4["kernels"].items()}, **stats(r4)}
        del m4, r4
        torch.cuda.empty_cache()

        log("[bench] generating DSA config (B8, 65536 tokens, indexer 64x128, top-2048)")
        d5 = wl.config5_dsa()
        r5 = bench_dsa(d5, timer, steps, warmup, torch, lib)
        ku = r5["kernels"]
        bi, fi = d5.indexer_bytes(), d5.indexer_flops()
        sel = d5.B * d5.topk
        fs = sel * 2 * d5.mla.H * (576 + 512)
        bs = sel * 576 * 2
        if cpu:
            import oracle
            want_idx = oracle.topk(oracle.indexer(d5.q_i, d5.w, d5.k_i, d5.seq_lens), d5.seq_lens, d5.topk)
            m = d5.mla
            rows = rows_sample(m.B * m.H, 48, 5)
            want, _ = oracle.mla(m.q, m.latent, idx=want_idx, scale=m.scale, rows=rows)
            e5 = err_record(r5["out"].float().cpu().reshape(-1, 512)[rows], want, 2e-2)
            e5["index_sets_bit_exact"] = bool(torch.equal(r5["idx"].cpu(), want_idx))
            errors["config5_" + d5.name] = e5
        result["workloads"]["dsa_top2048"] = {
            "step_us": round(r5["wall_ms"] * 1e3, 2),
            "indexer_GB/s": round(gbs(bi, ku["indexer_scores"]["avg_us"]), 1),
            "indexer_TFLOP/s": round(tflops(fi, ku["indexer_scores"]["avg_us"]), 1),
            "topk_us": ku["topk_select"]["avg_us"],
            "sparse_mla_TFLOP/s": round(tflops(fs, ku["sparse_mla_split"]["avg_us"]), 2),
            "sparse_mla_GB/s": round(gbs(bs, ku["sparse_mla_split"]["avg_us"]), 1),
            "sparse_mla_split": counter_fields("sparse_mla_split"),
            "indexer": counter_fields("indexer_bf16"),
            "copies": r5["copies"],
            "kernels_us": {k: v["avg_us"] for k, v in ku.items()}, **stats(r5),
            "indexer_fp8": {
                "indexer_us": r5["fp8"]["kernels"]["indexer_scores"]["avg_us"],
                "indexer_GB/s": round(gbs(bi // 2, r5["fp8"]["kernels"]["indexer_scores"]["avg_us"]), 1),
                "key_bytes_per_step": bi // 2,
                "indexer": counter_fields("indexer_fp8"),
                "indexer_topk_step_us": round(r5["fp8"]["wall_ms"] * 1e3, 2), **stats(r5["fp8"])}}
        del d5, r5
        torch.cuda.empty_cache()

        log("[bench] cache append (GQA K/V, MLA latent, indexer keys)")
        result["workloads"]["kv_append"] = bench_append(timer, steps, warmup, torch, lib)
        torch.cuda.empty_cache()

    if cpu:
        x1 = wl.config1_tiny_gqa()
        r1 = bench_gqa(x1, timer, min(steps, 20), 2, torch, lib)
        errors["config1_" + x1.name] = gqa_error(x1, r1, n_rows=x1.B * x1.Hq)
        result["cpu_baseline"] = cpu_baseline()
        result["cpu_baseline"]["max_error_vs_oracle"] = errors
    print(json.dumps(result), flush=True)


def read_ceiling(timer, torch, lib, nbytes, steps):
    """Best rate of the library's plain streaming-read probe over nbytes per
    launch, two buffers alternated (2 x nbytes > the Infinity Cache), over
    launch shapes: workgroups x loads in flight per thread."""
    nbytes = nbytes // 16 * 16
    bufs = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0") for _ in range(2)]
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launcher(grid, depth):
        return lambda i: check(lib, lib.dattn_stream_read_probe(ptr(bufs[i % 2]), nbytes, ptr(sink), grid,
                                                                 depth, stream))
    timer.ramp(launcher(1024, 8), 0)
    best, tried = None, []
    for grid in (512, 1024, 2048, 4096):
        for depth in (4, 8, 16):
            step = launcher(grid, depth)
            for i in range(4):
                step(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(steps):
                step(i)
            e1.record()
            torch.cuda.synchronize()
            us = 1e3 * e0.elapsed_time(e1) / steps
            rate = nbytes / (us * 1e-6) / 1e9
            tried.append([grid, depth, round(rate, 1)])
            if best is None or rate > best["GB/s"]:
                best = {"GB/s": round(rate, 1), "us": round(us, 2), "grid": grid, "loads_in_flight": depth}
    best.update({"bytes_per_launch": nbytes, "launches": steps,
                 "pct_of_hbm_peak": round(100 * best["GB/s"] / HBM_PEAK_GBS, 2),
                 "sweep_grid_depth_GBs": tried,
                 "probe": "dattn_stream_read_probe: 256-thread workgroups over contiguous ranges, "
                          "16-byte nontemporal loads"})
    del bufs
    return best


def calibrate_copy(torch, steps):
    """A plain device-to-device copy of 1 GiB: reads and writes exactly 1 GiB per
    launch, the reference that scales rocprofv3's FETCH_SIZE / WRITE_SIZE."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    us = 1e6 * (time.perf_counter() - t0) / steps
    print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "launches": steps, "avg_us": round(us, 2),
                      "GB/s_read+write": round(2 * n / (us * 1e-6) / 1e9, 1)}), flush=True)


def only(name, timer, steps, warmup, torch, lib, wl):
    if name == "gqa":
        x = wl.config2_llama3_8b_gqa()
        r = bench_gqa(x, timer, steps, warmup, torch, lib)
        r["kv_bytes_per_step"] = x.kv_bytes()
    elif name == "swa":
        x = wl.config3_swa_sinks()
        r = bench_gqa(x, timer, steps, warmup, torch, lib)
        r["kv_bytes_per_step"] = x.kv_bytes()
    elif name == "mla":
        m = wl.config4_mla()
        r = bench_mla(m, timer, steps, warmup, torch, lib)
        r["kv_bytes_per_step"], r["flops_per_step"] = m.kv_bytes(), m.flops()
    elif name == "append":
        r = bench_append(timer, steps, warmup, torch, lib)
    elif name == "layouts":
        r = bench_layouts(timer, steps, warmup, torch, lib, wl)
    elif name == "quest":
        x = wl.config2_llama3_8b_gqa()
        r = bench_quest(x, timer, steps, warmup, torch, lib, 128)
        summ, bnd, selb, unib = quest_bytes(x, 128, r.pop("selected"))
        r["bytes_per_step"] = summ + bnd + unib
        r["kv_bytes_per_head_sum"], r["kv_bytes_union_per_kv_head"] = selb, unib
    elif name == "read":
        r = read_ceiling(timer, torch, lib, wl.config2_llama3_8b_gqa().kv_bytes(), steps)
    else:
        d = wl.config5_dsa()
        r = bench_dsa(d, timer, steps, warmup, torch, lib)
        r["indexer_bytes_per_step"] = d.indexer_bytes()
    for k in ("out", "lse", "idx"):
        r.pop(k, None)
    r["workload"] = name
    print(json.dumps(r), flush=True)


def bench_layouts(timer, steps, warmup, torch, lib, wl):
    """Other head layouts at config 2's K/V bytes: 64 q / 8 KV heads at D128
    (eight heads per KV head), and D64 over twice the tokens."""
    out = {}
    for hq, d, s_len in ((64, 128, 8192), (64, 64, 16384), (32, 64, 16384)):
        name = f"gqa_{hq}q8kv_d{d}_b16_s{s_len}_paged16"
        log(f"[bench] generating {name}")
        xh = wl.make_gqa(B=16, Hq=hq, Hkv=8, D=d, seq_lens=[s_len] * 16, dtype=torch.bfloat16,
                         page_size=16, seed=3, name=name)
        bh = xh.kv_bytes()
        rh = bench_gqa(xh, timer, steps, warmup, torch, lib)
        out[name] = {
            "step_us": round(rh["wall_ms"] * 1e3, 2),
            "GB/s": round(bh / (rh["wall_ms"] * 1e-3) / 1e9, 1),
            "split_kernel_GB/s": round(gbs(bh, rh["kernels"]["gqa_split"]["avg_us"]), 1),
            "kv_bytes_per_step": bh,
            "kernels_us": {k: v["avg_us"] for k, v in rh["kernels"].items()}, **stats(rh)}
        del xh, rh
        torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(target_s=15.0, max_passes=500):
    """The oracle on the host cores, on the headline workload: whole passes
    repeated until about target_s seconds of CPU work (a bounded sample)."""
    import oracle
    from decode_attention_kv_flash_amd import workloads as wl
    x = wl.config2_llama3_8b_gqa()
    nbytes = x.kv_bytes()
    log(f"[bench] cpu oracle on the gqa workload, {oracle.threads()} threads")
    reps, total = 0, 0.0
    while total < target_s and reps < max_passes:
        t0 = time.perf_counter()
        oracle.gqa(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
        total += time.perf_counter() - t0
        reps += 1
    value = nbytes * reps / total / 1e9
    return {"value": round(value, 3), "unit": "GB/s", "cores": oracle.threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"full gqa workload ({x.B * x.Hq} rows x {int(x.seq_lens[0])} tokens, "
                      f"{nbytes} KV bytes) x {reps} passes, {total:.1f} s"}

if __name__ == "__main__":
    main()
