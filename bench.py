#!/usr/bin/env python3
"""Benchmark of single-token decode attention over a KV cache on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--quick] [--no-cpu-baseline]

Prints ONE JSON line on stdout.  The headline `value` is the KV bytes the
Llama-3-8B-shaped GQA layer must read (B16, 32/8 heads, D128, 8192 tokens,
paged 16, bf16) divided by the wall time of one decode_attn_gqa call (split
kernel + log-sum-exp combine), K calls timed back to back with inputs resident
in HBM.  The other workloads (window + sinks, MLA, DSA, Quest page selection,
cache append) are reported under
"workloads".  A step is one call of the hot path on one batch; buffers rotate
over copies whose total exceeds 1 GiB so no step reads another's data from
the 256 MB Infinity Cache.

`roofline` covers the dominant kernel (gqa_split): algorithmic bytes per
launch over its average duration, measured with HIP events the library
records around each launch on the same stream, in a second pass of the same
K steps (the first pass, without events, gives the step time).  `cpu_baseline` is the CPU
oracle (plain fp64 C, OpenMP over rows) timed on this host on the same
workload.
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


def copies_for(nbytes):
    return max(1, min(8, math.ceil(ROTATE_BYTES / max(1, nbytes))))


def sha256_of(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def counter_traffic(kernel, source):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, "decode_attention_kv_flash_amd", "csrc", source)
    if rec.get("source_sha256") != sha256_of(src):
        return None
    return rec.get("hbm_bytes_per_launch")


class Timer:
    def __init__(self, api, torch):
        self.api, self.torch = api, torch

    def run(self, step, steps, warmup, kernels):
        """K timed steps, twice: first plain (the step time), then with the
        library's per-kernel HIP events enabled (kernel durations)."""
        torch, api = self.torch, self.api
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
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
        return {"wall_ms": 1e3 * (t1 - t0) / steps, "event_ms": e0.elapsed_time(e1) / steps,
                "kernels": per_kernel}


def check(lib, rc):
    if rc != 0:
        raise RuntimeError(lib.dattn_last_error().decode())


def bench_gqa(x, timer, steps, warmup, torch, lib, sink_logits=None):
    """decode_attn_gqa on a (paged) GQA workload (decode_attn_gqa_sink when
    sink_logits, fp32 [Hq], is given); returns the timing record."""
    dev = torch.device("cuda:0")
    q, sl = x.q.to(dev), x.seq_lens.to(dev)
    pt = x.page_table.to(dev) if x.page_table is not None else None
    kv_bytes_alloc = 2 * x.k_cache.numel() * x.k_cache.element_size()
    R = copies_for(kv_bytes_alloc)
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
    return rec


def bench_mla(m, timer, steps, warmup, torch, lib):
    dev = torch.device("cuda:0")
    q, sl = m.q.to(dev), m.seq_lens.to(dev)
    R = copies_for(m.latent.numel() * 2)
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
    return rec


def bench_dsa(d, timer, steps, warmup, torch, lib):
    """Indexer + top-k over the full context, then sparse MLA over the selection."""
    dev = torch.device("cuda:0")
    m = d.mla
    B, Hi, Di = d.q_i.shape
    S = d.k_i.shape[1]
    R = copies_for(d.k_i.numel() * 2)
    qi, w, sl = d.q_i.to(dev), d.w.to(dev), d.seq_lens.to(dev)
    ki = [d.k_i.to(dev) for _ in range(R)]
    q, lat = m.q.to(dev), m.latent.to(dev)
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
    a2 = (ptr(q), ptr(lat), ptr(idx), d.topk, ptr(out), ptr(lse), B, m.H, 512, 64, m.S_max, 1,
          ctypes.c_float(m.scale), 0, ptr(ws), nbytes, stream)

    def step(i):
        check(lib, lib.dsa_indexer_topk(*a1[i % R]))
        check(lib, lib.sparse_mla_attn(*a2))

    rec = timer.run(step, steps, warmup, ["indexer_scores", "topk_select", "sparse_mla_split",
                                          "lse_combine"])
    rec["copies"] = R
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
    R = copies_for(2 * x.k_cache.numel() * x.k_cache.element_size())
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the GPU's clocks take ~20 ms of sustained work to ramp up after idling
    # (input generation runs on the CPU); 300 calls cover that
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--only", choices=["gqa", "swa", "mla", "dsa", "append", "quest"],
                    help="time one workload and print its record (for profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="time a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
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
    timer = Timer(api, torch)
    steps, warmup = args.steps, args.warmup
    if args.calibrate_copy:
        calibrate_copy(torch, steps)
        return
    if args.only:
        only(args.only, timer, steps, warmup, torch, lib, wl)
        return

    # ---- headline: Llama-3-8B-shaped GQA layer --------------------------------
    log("[bench] generating gqa config (B16, 32/8 heads, D128, 8192 tokens, paged 16, bf16)")
    x2 = wl.config2_llama3_8b_gqa()
    bytes2 = x2.kv_bytes()
    flops2 = x2.attended_tokens() * 4 * x2.Hq * x2.D  # 4 S n_h d_h per sequence
    r2 = bench_gqa(x2, timer, steps, warmup, torch, lib)
    split_us = r2["kernels"]["gqa_split"]["avg_us"]
    log(f"[bench] gqa: {r2['wall_ms']*1e3:.1f} us/step wall, split kernel {split_us:.1f} us")
    value = bytes2 / (r2["wall_ms"] * 1e-3) / 1e9
    achieved = gbs(bytes2, split_us)
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
        },
        "roofline": {
            "kernel": "gqa_split",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": counter_traffic("gqa_split", "gqa_decode.hip"),
            "algorithmic_bytes_per_launch": bytes2,
            "avg_launch_us": round(split_us, 2),
        },
        "workloads": {
            "gqa_llama3_8b": {"step_us": round(r2["wall_ms"] * 1e3, 2), "GB/s": round(value, 1),
                              "TFLOP/s": round(flops2 / (r2["wall_ms"] * 1e-3) / 1e12, 3),
                              "kernels_us": {k: v["avg_us"] for k, v in r2["kernels"].items()}},
        },
    }
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
            "dense_step_us": round(r2["wall_ms"] * 1e3, 2),
            "bytes_per_step": summ + bnd + unib,
            "GB/s": round((summ + bnd + unib) / (rq["wall_ms"] * 1e-3) / 1e9, 1),
            "kv_bytes_per_head_sum": selb,
            "kv_bytes_union_per_kv_head": unib,
            "bounds_GB/s": round(gbs(summ, kq["quest_bounds"]["avg_us"]), 1),
            "attention_GB/s": round(gbs(unib, kq["gqa_split"]["avg_us"]), 1),
            "topk_us": kq["topk_select"]["avg_us"],
            "kernels_us": {k: v["avg_us"] for k, v in kq.items()},
            "minmax_all_blocks_us": round(mm_us, 2),
            "minmax_all_blocks_GB/s": round(gbs(kbytes, mm_us), 1),
            "minmax_one_block_us": round(rq["minmax_one_block"]["kernels"]["quest_minmax"]["avg_us"], 2)}
    del x2

    if not args.quick:
        log("[bench] generating window+sinks config (B32, lens U[4096,32768], W4096 + 4 sinks)")
        x3 = wl.config3_swa_sinks()
        b3 = x3.kv_bytes()
        r3 = bench_gqa(x3, timer, steps, warmup, torch, lib)
        result["workloads"]["swa4096_sinks4"] = {
            "step_us": round(r3["wall_ms"] * 1e3, 2),
            "GB/s": round(b3 / (r3["wall_ms"] * 1e-3) / 1e9, 1),
            "split_kernel_GB/s": round(gbs(b3, r3["kernels"]["gqa_split"]["avg_us"]), 1),
            "kv_bytes_per_step": b3,
            "kernels_us": {k: v["avg_us"] for k, v in r3["kernels"].items()}}
        # the same workload with an explicit sink logit per head
        sk = torch.linspace(-2.0, 2.0, x3.Hq, dtype=torch.float32)
        r3s = bench_gqa(x3, timer, steps, warmup, torch, lib, sink_logits=sk)
        result["workloads"]["swa4096_sinks4_sink_logits"] = {
            "step_us": round(r3s["wall_ms"] * 1e3, 2),
            "GB/s": round(b3 / (r3s["wall_ms"] * 1e-3) / 1e9, 1),
            "split_kernel_GB/s": round(gbs(b3, r3s["kernels"]["gqa_split"]["avg_us"]), 1),
            "kv_bytes_per_step": b3,
            "kernels_us": {k: v["avg_us"] for k, v in r3s["kernels"].items()}}
        del x3
        torch.cuda.empty_cache()

        # other head layouts at config 2's K/V bytes: 64 q / 8 KV heads at D128
        # (eight heads per KV head), and D64 over twice the tokens
        result["workloads"]["gqa_head_layouts"] = {}
        for hq, d, s_len in ((64, 128, 8192), (64, 64, 16384), (32, 64, 16384)):
            name = f"gqa_{hq}q8kv_d{d}_b16_s{s_len}_paged16"
            log(f"[bench] generating {name}")
            xh = wl.make_gqa(B=16, Hq=hq, Hkv=8, D=d, seq_lens=[s_len] * 16, dtype=torch.bfloat16,
                             page_size=16, seed=3, name=name)
            bh = xh.kv_bytes()
            rh = bench_gqa(xh, timer, steps, warmup, torch, lib)
            result["workloads"]["gqa_head_layouts"][name] = {
                "step_us": round(rh["wall_ms"] * 1e3, 2),
                "GB/s": round(bh / (rh["wall_ms"] * 1e-3) / 1e9, 1),
                "split_kernel_GB/s": round(gbs(bh, rh["kernels"]["gqa_split"]["avg_us"]), 1),
                "kv_bytes_per_step": bh,
                "kernels_us": {k: v["avg_us"] for k, v in rh["kernels"].items()}}
            del xh
            torch.cuda.empty_cache()

        log("[bench] generating MLA config (B32, H128, latent 576, 16384 tokens)")
        m4 = wl.config4_mla()
        r4 = bench_mla(m4, timer, steps, warmup, torch, lib)
        b4, f4 = m4.kv_bytes(), m4.flops()
        us4 = r4["kernels"]["mla_split"]["avg_us"]
        result["workloads"]["mla_dsv3"] = {
            "step_us": round(r4["wall_ms"] * 1e3, 2),
            "TFLOP/s": round(f4 / (r4["wall_ms"] * 1e-3) / 1e12, 1),
            "GB/s": round(b4 / (r4["wall_ms"] * 1e-3) / 1e9, 1),
            "split_kernel_TFLOP/s": round(tflops(f4, us4), 1),
            "mfma_frac_of_bf16_peak": round(tflops(f4, us4) / BF16_PEAK_TFLOPS, 4),
            "split_kernel_hbm_frac": round(gbs(b4, us4) / HBM_PEAK_GBS, 4),
            "kernels_us": {k: v["avg_us"] for k, v in r4["kernels"].items()}}
        del m4
        torch.cuda.empty_cache()

        log("[bench] generating DSA config (B8, 65536 tokens, indexer 64x128, top-2048)")
        d5 = wl.config5_dsa()
        r5 = bench_dsa(d5, timer, steps, warmup, torch, lib)
        ku = r5["kernels"]
        bi, fi = d5.indexer_bytes(), d5.indexer_flops()
        sel = d5.B * d5.topk
        fs = sel * 2 * d5.mla.H * (576 + 512)
        bs = sel * 576 * 2
        result["workloads"]["dsa_top2048"] = {
            "step_us": round(r5["wall_ms"] * 1e3, 2),
            "indexer_GB/s": round(gbs(bi, ku["indexer_scores"]["avg_us"]), 1),
            "indexer_TFLOP/s": round(tflops(fi, ku["indexer_scores"]["avg_us"]), 1),
            "topk_us": ku["topk_select"]["avg_us"],
            "sparse_mla_TFLOP/s": round(tflops(fs, ku["sparse_mla_split"]["avg_us"]), 2),
            "sparse_mla_GB/s": round(gbs(bs, ku["sparse_mla_split"]["avg_us"]), 1),
            "kernels_us": {k: v["avg_us"] for k, v in ku.items()},
            "indexer_fp8": {
                "indexer_us": r5["fp8"]["kernels"]["indexer_scores"]["avg_us"],
                "indexer_GB/s": round(gbs(bi // 2, r5["fp8"]["kernels"]["indexer_scores"]["avg_us"]), 1),
                "key_bytes_per_step": bi // 2,
                "indexer_topk_step_us": round(r5["fp8"]["wall_ms"] * 1e3, 2)}}
        del d5
        torch.cuda.empty_cache()

        log("[bench] cache append (GQA K/V, MLA latent, indexer keys)")
        result["workloads"]["kv_append"] = bench_append(timer, steps, warmup, torch, lib)
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


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
    elif name == "quest":
        x = wl.config2_llama3_8b_gqa()
        r = bench_quest(x, timer, steps, warmup, torch, lib, 128)
        summ, bnd, selb, unib = quest_bytes(x, 128, r.pop("selected"))
        r["bytes_per_step"] = summ + bnd + unib
        r["kv_bytes_per_head_sum"], r["kv_bytes_union_per_kv_head"] = selb, unib
    else:
        d = wl.config5_dsa()
        r = bench_dsa(d, timer, steps, warmup, torch, lib)
        r["indexer_bytes_per_step"] = d.indexer_bytes()
    r["workload"] = name
    print(json.dumps(r), flush=True)


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
            "sample": f"full gqa workload ({x.B * x.Hq} rows x {int(x.seq_lens[0])} tokens, "
                      f"{nbytes} KV bytes) x {reps} passes, {total:.1f} s"}

if __name__ == "__main__":
    main()
