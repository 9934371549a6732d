"""Benchmark: one decode step of absorbed MLA (absorb_q, cache_append, decode,
up_v) over a paged latent KV cache on one MI355X.

Default workload: DeepSeek-V2 shapes (n_h = 128, d_h = 128, d_c = 512,
d_R = 64), batch 16, 4096 cached tokens per sequence, 64-token pages, bf16.
Each step appends the current token of every sequence, then attends over its
whole cache (history plus current).  Caches and weights are replicated and
rotated per step (like consecutive layers) so that the 256 MB Infinity Cache
cannot hold the working set; every input is resident in HBM before timing.

Prints one JSON line (see the repository documentation for the fields).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode: latent-KV GB/s + TFLOP/s as % of roofline, 128 heads, B=16×4K bf16"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="v2_b16_4k")
    p.add_argument("--splits", type=int, default=0)
    p.add_argument("--min-replica-mb", type=float, default=600.0)
    p.add_argument("--cpu-sample-s", type=float, default=10.0,
                   help="seconds of oracle work for the CPU baseline (whole sequences, in batch order)")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the fused-projection and multi-query measurements (profiling runs)")
    p.add_argument("--graph", action="store_true",
                   help="replay each step from a captured HIP graph (one graph per cache replica)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB three times (calibrates the "
                        "FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    return p.parse_args()


# Kernel sources the stored HBM-traffic measurement depends on; the stored
# figure is reported only while their hash matches.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
TRAFFIC_SOURCES = ["mla_latent_kv_38_amd/csrc/k_decode_h64w.hip", "mla_latent_kv_38_amd/csrc/k_decode_e4m3_h64.hip",
                   "mla_latent_kv_38_amd/csrc/k_decode_fp8.hip", "mla_latent_kv_38_amd/csrc/mla_device.h"]


def source_hash(paths):
    """Hash of the code in the given C++ sources: comments and whitespace are
    left out, so that only a change to the code itself retires a stored
    measurement."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload):
    """HBM bytes per decode call measured with rocprofv3 counters (see the
    profiles directory), or None if absent or taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(workload)
    if not rec or rec.get("source_hash") != source_hash(TRAFFIC_SOURCES):
        return None
    return rec.get("bytes_per_call")


def copy_probe(mib):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 3}))


EXTRA_WORKLOADS = ("ragged_b64", "long_b4_128k", "fp8_h16_b128")


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              f"multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch

    import mla_inputs as W
    import mla_latent_kv_38_amd as mla

    dev = torch.device("cuda:0")
    res, w, row_bytes = measure(args, W, mla, dev, args.workload, args.steps, args.warmup, extras=not args.no_extras)
    others = {}
    if not args.no_extras and args.workload == "v2_b16_4k":
        # the other workloads, decode-step lines of their own (fewer steps)
        for name in EXTRA_WORKLOADS:
            r, _, _ = measure(args, W, mla, dev, name, min(args.steps, 30), min(args.warmup, 5), extras=False)
            others[name] = {k: r[k] for k in ("value", "unit", "ms_per_step", "decode_us", "call_us", "roofline",
                                              "config")}
            torch.cuda.empty_cache()
    # the probes last: a second of full-chip MFMA load leaves the clocks lower
    # for what runs right after it
    peaks = achievable_peaks(mla, dev)
    _against_achievable(res["roofline"], peaks)
    res["achievable_peaks"] = peaks
    for r in others.values():
        _against_achievable(r["roofline"], peaks)
    if others:
        res["workloads"] = others
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_s, row_bytes)
    print(json.dumps(res))


def _against_achievable(roof, peaks):
    """The decode's rate as a fraction of what the probes achieved too."""
    a = peaks["hbm_read_GBps"] if roof["bound"] == "hbm" else peaks["bf16_mfma_TFLOPs"]
    roof["achievable_peak"] = a
    roof["frac_of_achievable"] = round(roof["achieved"] / a, 4)


def achievable_peaks(mla, dev, read_gib=2, mfma_iters=2000, mfma_wgs=2048, reps=5):
    """What the chip achieves on a plain streaming read of read_gib GiB (one
    pass, 2048 workgroups, 16-B nontemporal loads) and on a plain bf16 MFMA
    loop (mfma_wgs workgroups of 4 waves, four independent 32x32x16 chains
    each), timed with events on the launch stream, best of `reps`."""
    import ctypes

    import torch
    lib = mla._lib.lib()
    stream = torch.cuda.current_stream()
    n = read_gib << 30
    buf = torch.ones(n // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(max(8192, 4 * mfma_wgs), dtype=torch.uint8, device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def best(launch):
        launch()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts)

    def rd():
        mla._lib.check(lib.mla_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()),
                                                 sp), "mla_probe_stream_read")

    def mm():
        mla._lib.check(lib.mla_probe_mfma_bf16(mfma_iters, mfma_wgs, ctypes.c_void_p(sink.data_ptr()), sp),
                       "mla_probe_mfma_bf16")
    t_rd = best(rd)
    t_mm = best(mm)
    flops = 16.0 * 32768 * mfma_iters * mfma_wgs
    del buf
    torch.cuda.empty_cache()
    return {"hbm_read_GBps": round(n / t_rd / 1e9, 1), "read_bytes": n,
            "bf16_mfma_TFLOPs": round(flops / t_mm / 1e12, 1), "mfma_flops": flops,
            "spec": {"hbm_GBps": HBM_PEAK_GBPS, "bf16_mfma_TFLOPs": BF16_PEAK_TFLOPS}}


def measure(args, W, mla, dev, name, steps, warmup, extras):
    """One workload's decode steps; returns (result line fields, workload,
    cache row bytes)."""
    import torch
    w = W.make(name)
    B, nh, D = w.B, w.n_h, w.D
    act = torch.bfloat16 if w.act == "bf16" else torch.float32
    d = mla.make_dims(w.n_h, w.d_h, w.d_c, w.d_R, w.block_size, act=w.act, kv=w.kv,
                      softmax_scale=w.scale, rope_base=w.rope_base)
    esz = 1 if w.kv == "e4m3" else (2 if w.kv == "bf16" else 4)
    row_bytes = D * esz + (4 if w.kv == "e4m3" else 0)
    cache_bytes = w.num_pages * w.block_size * row_bytes
    weight_bytes = 2 * nh * w.d_h * w.d_c * (2 if w.act == "bf16" else 4)
    R = max(1, math.ceil(args.min_replica_mb * 1e6 / (cache_bytes + weight_bytes)))

    def g(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)

    # history (all but the current token) goes into every replica's cache
    hist_c = np.concatenate([w.c_kv[b][:-1] for b in range(B)])
    hist_k = np.concatenate([w.k_r[b][:-1] for b in range(B)])
    hist_pos = np.concatenate([np.arange(w.lens[b] - 1) for b in range(B)]).astype(np.int32)
    hist_slot = np.concatenate([w.slots(b, 0, int(w.lens[b]) - 1) for b in range(B)])
    cur_c = np.stack([w.c_kv[b][-1] for b in range(B)])
    cur_k = np.stack([w.k_r[b][-1] for b in range(B)])
    cur_pos = (w.lens - 1).astype(np.int32)
    cur_slot = np.array([w.slots(b, int(w.lens[b]) - 1)[0] for b in range(B)], dtype=np.int64)

    t_hist = (g(hist_c, act), g(hist_k, act), g(hist_pos, torch.int32), g(hist_slot, torch.int64))
    cur = (g(cur_c, act), g(cur_k, act), g(cur_pos, torch.int32), g(cur_slot, torch.int64))
    q_c, q_r = g(w.q_c, act), g(w.q_r, act)
    q_pos = g(w.q_pos, torch.int32)
    bt, lens = g(w.block_table, torch.int32), g(w.lens, torch.int32)
    w_uk0, w_uv0 = g(w.w_uk, act), g(w.w_uv, act)

    reps = []
    fill_ms = []
    for r in range(R):
        if w.kv == "e4m3":
            cache = torch.zeros((w.num_pages, w.block_size, D), dtype=torch.uint8, device=dev)
            scale = torch.ones((w.num_pages, w.block_size), dtype=torch.float32, device=dev)
        else:
            cache = torch.zeros((w.num_pages, w.block_size, D), dtype=act, device=dev)
            scale = None
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        mla.cache_append(d, *t_hist, cache, scale)
        e1.record()
        torch.cuda.synchronize()
        fill_ms.append(e0.elapsed_time(e1))
        reps.append(dict(cache=cache, scale=scale, w_uk=w_uk0.clone(), w_uv=w_uv0.clone()))
    ws = torch.empty(mla.decode_workspace_bytes(d, B, args.splits), dtype=torch.uint8, device=dev)
    q_abs = torch.empty((B, nh, D), dtype=act, device=dev)
    o_lat = torch.empty((B, nh, w.d_c), dtype=act, device=dev)
    lse = torch.empty((B, nh), dtype=torch.float32, device=dev)
    out = torch.empty((B, nh, w.d_h), dtype=act, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        rp = reps[i % R]
        rec = (lambda k: ev[k].record(stream) if ev[k] is not None else None) if ev is not None else (lambda k: None)
        rec(0)
        # absorb_q and the current token's append are independent: one call
        # (one launch for these shapes); mla_absorb_q + mla_cache_append
        # compute the same bytes
        mla.absorb_q_append(d, q_c, q_r, q_pos, rp["w_uk"], *cur, rp["cache"], rp["scale"], q_abs=q_abs)
        rec(1)
        rec(2)
        mla.decode(d, q_abs, rp["cache"], bt, lens, kv_scale=rp["scale"], num_splits=args.splits,
                   workspace=ws, o_lat=o_lat, lse=lse)
        rec(3)
        mla.up_v(d, o_lat, rp["w_uv"], out)
        rec(4)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    graphs = None
    if args.graph:
        # the library allocates nothing and issues no memset, so a step captures
        # as four kernel launches (five with the split-KV merge) per replica
        graphs = []
        for r in range(R):
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gph):
                step(r)
            graphs.append(gph)
        for i in range(warmup):
            graphs[i % R].replay()
        torch.cuda.synchronize()

    # timed region: K whole steps; events only around the decode call (the
    # roofline kernel), on the stream the library launches on
    new_ev = lambda: torch.cuda.Event(enable_timing=True)
    t0, t1 = new_ev(), new_ev()
    dec_evs = [[None, None, new_ev(), new_ev(), None] for _ in range(steps)]
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        if graphs is not None:
            graphs[i % R].replay()
        else:
            step(i, dec_evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / steps
    dec_us = None if graphs is not None else float(np.mean([e[2].elapsed_time(e[3]) for e in dec_evs]) * 1e3)

    # per-call breakdown: a second, untimed pass with an event between calls
    evs = [[new_ev() for _ in range(5)] for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    call_us = {name: float(np.mean([e[k].elapsed_time(e[k + 1]) for e in evs]) * 1e3)
               for k, name in ((0, "absorb_q_append"), (2, "decode"), (3, "up_v"))}
    if dec_us is None:                   # graph replay: the decode call is timed in the eager pass
        dec_us = call_us["decode"]

    kvp = mq = e8 = None
    if extras:
        kvp = kv_project_measure(mla, d, w, dev, B, args.min_replica_mb)
        mq = multi_query_measure(mla, d, w, dev, reps, bt, lens, act, iters=20)
        if w.kv == "bf16" and w.act == "bf16" and w.n_h % 64 == 0:
            e8 = e4m3_measure(mla, w, dev, t_hist, cur, q_abs, bt, lens, args.min_replica_mb)

    # algorithmic work of one decode call
    toks = int(w.lens.sum())
    kv_bytes = toks * row_bytes
    q_bytes = B * nh * D * (2 if w.act == "bf16" else 4)
    o_bytes = B * nh * w.d_c * (2 if w.act == "bf16" else 4) + B * nh * 4
    dec_bytes = kv_bytes + q_bytes + o_bytes
    flops_tok = 2 * nh * D + 2 * nh * w.d_c
    dec_flops = toks * flops_tok
    ach_gbps = dec_bytes / (dec_us * 1e-6) / 1e9
    ach_tflops = dec_flops / (dec_us * 1e-6) / 1e12
    ai = dec_flops / dec_bytes
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if ai < ridge:
        roof = dict(bound="hbm", achieved=round(ach_gbps, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(ach_gbps / HBM_PEAK_GBPS, 4))
    else:
        roof = dict(bound="mfma", achieved=round(ach_tflops, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(ach_tflops / BF16_PEAK_TFLOPS, 4))
    roof.update(traffic=stored_traffic(name), kernel="mla_decode (split + combine)",
                algorithmic_bytes=dec_bytes,
                algorithmic_flops=dec_flops, avg_us=round(dec_us, 3),
                tflops=round(ach_tflops, 1), tflops_frac=round(ach_tflops / BF16_PEAK_TFLOPS, 4))

    step_kv_gbps = kv_bytes / (ms_step * 1e-3) / 1e9

    res = {
        "metric": METRIC, "value": round(step_kv_gbps, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.act,
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "seq_len": int(w.lens.max()),
                   "total_tokens": toks, "n_heads": nh, "d_head": w.d_h, "d_latent": w.d_c,
                   "d_rope": w.d_R, "block_size": w.block_size, "kv_dtype": w.kv,
                   "replicas": R, "num_splits": args.splits,
                   "launch": "graph" if graphs is not None else "eager"},
        "steps_per_s": round(1e3 / ms_step, 1),
        "step_tflops": round(dec_flops / (ms_step * 1e-3) / 1e12, 1),
        "decode_us": round(dec_us, 3),
        "call_us": {k: round(v, 3) for k, v in call_us.items()},
        "roofline": roof,
        "cache_fill_GBps": round(cache_bytes / (np.median(fill_ms) * 1e-3) / 1e9, 1),
        "kv_project": kvp,
        "multi_query": mq,
        "e4m3_cache": e8,
    }

    del reps, ws
    return res, w, row_bytes


def kv_project_measure(mla, d, w, dev, T, min_mb, d_model=5120, iters=50):
    """mla_kv_project_append for the step's T new tokens (d_model = 5120, the
    DeepSeek-V2 hidden width): mean call time over calls that rotate through
    enough copies of W_DKV / W_KR (random, bf16) to exceed the MALL, replayed
    from a captured graph, and its HBM rate on the algorithmic bytes (weights
    once, hidden states, rows written)."""
    import torch
    if w.act != "bf16":
        return None
    wb = (w.d_c + w.d_R) * d_model * 2
    R = max(1, math.ceil(min_mb * 1e6 / wb))
    gen = torch.Generator(device=dev).manual_seed(7)
    mk = lambda r, c: (torch.randn((r, c), generator=gen, device=dev) / math.sqrt(c)).to(torch.bfloat16)
    ws_w = [(mk(w.d_c, d_model), mk(w.d_R, d_model)) for _ in range(R)]
    h = torch.randn((T, d_model), generator=gen, device=dev).to(torch.bfloat16)
    pages = (T + w.block_size - 1) // w.block_size
    if w.kv == "e4m3":
        cache = torch.zeros((pages, w.block_size, w.D), dtype=torch.uint8, device=dev)
        scale = torch.ones((pages, w.block_size), dtype=torch.float32, device=dev)
    else:
        cache = torch.zeros((pages, w.block_size, w.D), dtype=torch.bfloat16, device=dev)
        scale = None
    pos = torch.arange(T, dtype=torch.int32, device=dev)
    slot = torch.arange(T, dtype=torch.int64, device=dev)
    ws = torch.empty(mla.kv_project_workspace_bytes(d, T, d_model), dtype=torch.uint8, device=dev)
    for i in range(5):
        mla.kv_project_append(d, h, *ws_w[i % R], pos, slot, cache, scale, workspace=ws)
    torch.cuda.synchronize()
    # one captured graph calls it once per weight copy, so the timing is the
    # device's (two kernels per call), not the Python loop's
    gph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gph):
        for i in range(R):
            mla.kv_project_append(d, h, *ws_w[i], pos, slot, cache, scale, workspace=ws)
    gph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(1, iters // R + 1)
    e0.record(stream)
    for _ in range(reps):
        gph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / (reps * R) * 1e3
    esz = 1 if w.kv == "e4m3" else 2
    nbytes = wb + T * d_model * 2 + T * (w.D * esz + (4 if w.kv == "e4m3" else 0))
    gbps = nbytes / (us * 1e-6) / 1e9
    del ws_w
    return {"tokens": T, "d_model": d_model, "us": round(us, 3), "algorithmic_bytes": nbytes,
            "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4), "weight_copies": R,
            "launch": "graph"}


def e4m3_measure(mla, w, dev, t_hist, cur, q_abs, bt, lens, min_mb, iters=50):
    """The same decode call with the cache stored as E4M3 rows and one float32
    scale per row (same history and current rows, same queries): mean call
    time over replicas rotated per call, and the rate against the bf16 MFMA
    peak, which bounds it (the arithmetic runs on bf16 MFMA after exact code
    conversion: 2 n_h (576 + 512) flops per 580-byte row, 480 flop/B at 128
    heads, above the ridge)."""
    import torch
    B, nh, D = w.B, w.n_h, w.D
    d8 = mla.make_dims(nh, w.d_h, w.d_c, w.d_R, w.block_size, act=w.act, kv="e4m3",
                       softmax_scale=w.scale, rope_base=w.rope_base)
    row = D + 4
    cache_bytes = w.num_pages * w.block_size * row
    R = max(2, math.ceil(min_mb * 1e6 / cache_bytes))
    reps = []
    for _ in range(R):
        c = torch.zeros((w.num_pages, w.block_size, D), dtype=torch.uint8, device=dev)
        sc = torch.ones((w.num_pages, w.block_size), dtype=torch.float32, device=dev)
        mla.cache_append(d8, *t_hist, c, sc)
        mla.cache_append(d8, *cur, c, sc)
        reps.append((c, sc))
    ws = torch.empty(mla.decode_workspace_bytes(d8, B, 0), dtype=torch.uint8, device=dev)
    o = torch.empty((B, nh, w.d_c), dtype=q_abs.dtype, device=dev)
    l = torch.empty((B, nh), dtype=torch.float32, device=dev)
    for i in range(3):
        mla.decode(d8, q_abs, reps[i % R][0], bt, lens, kv_scale=reps[i % R][1], workspace=ws, o_lat=o, lse=l)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    for i in range(iters):
        evs[i][0].record(stream)
        mla.decode(d8, q_abs, reps[i % R][0], bt, lens, kv_scale=reps[i % R][1], workspace=ws, o_lat=o, lse=l)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in evs]) * 1e3)
    toks = int(w.lens.sum())
    flops = toks * (2 * nh * D + 2 * nh * w.d_c)
    nbytes = toks * row + B * nh * D * 2 + B * nh * w.d_c * 2 + B * nh * 4
    tfl = flops / (us * 1e-6) / 1e12
    return {"kv_dtype": "e4m3", "us": round(us, 3), "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "bound": "mfma", "TFLOPs": round(tfl, 1), "frac": round(tfl / BF16_PEAK_TFLOPS, 4),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "replicas": R,
            "traffic": stored_traffic(w.name + "_e4m3")}


def multi_query_measure(mla, d, w, dev, reps, bt, lens, act, q_len=4, iters=20):
    """mla_decode_multi with q_len new query tokens per sequence (the last
    q_len rows of each sequence are theirs) on the same caches: mean call
    time, the HBM rate on the algorithmic bytes (every latent row once, the
    queries, the outputs) and the MFMA rate on the algorithmic flops (each
    query over its own rows); `frac` is against whichever bounds the call
    (at 128 heads and q_len 4 the flops per byte are above the bf16 ridge,
    so the MFMA does)."""
    import torch
    B, nh, D = w.B, w.n_h, w.D
    gen = torch.Generator(device=dev).manual_seed(11)
    q_abs = torch.randn((B, q_len, nh, D), generator=gen, device=dev).to(act)
    ws = torch.empty(int(mla._lib.lib().mla_decode_multi_workspace_bytes(__import__("ctypes").byref(d), B,
                                                                          q_len, 0)),
                     dtype=torch.uint8, device=dev)
    o = torch.empty((B, q_len, nh, w.d_c), dtype=act, device=dev)
    l = torch.empty((B, q_len, nh), dtype=torch.float32, device=dev)
    R = len(reps)
    for i in range(3):
        rp = reps[i % R]
        mla.decode_multi(d, q_abs, rp["cache"], bt, lens, kv_scale=rp["scale"], workspace=ws, o_lat=o, lse=l)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(iters):
        rp = reps[i % R]
        mla.decode_multi(d, q_abs, rp["cache"], bt, lens, kv_scale=rp["scale"], workspace=ws, o_lat=o, lse=l)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / iters * 1e3
    esz = 1 if w.kv == "e4m3" else (2 if w.kv == "bf16" else 4)
    asz = 2 if w.act == "bf16" else 4
    nbytes = int(w.lens.sum()) * (D * esz + (4 if w.kv == "e4m3" else 0)) + B * q_len * nh * (D + w.d_c) * asz
    # query i of sequence b attends to its first L_b - q_len + 1 + i rows
    rows = sum(max(0, int(L) - q_len + 1 + i) for L in w.lens for i in range(q_len))
    flops = rows * (2 * nh * D + 2 * nh * w.d_c)
    gbps = nbytes / (us * 1e-6) / 1e9
    tfl = flops / (us * 1e-6) / 1e12
    mfma_bound = flops / nbytes > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    return {"q_len": q_len, "us": round(us, 3), "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "GBps": round(gbps, 1), "TFLOPs": round(tfl, 1), "bound": "mfma" if mfma_bound else "hbm",
            "frac": round(tfl / BF16_PEAK_TFLOPS if mfma_bound else gbps / HBM_PEAK_GBPS, 4)}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_rate(O, w, seconds):
    """Whole-sequence oracle decodes in batch order (wrapping round) until
    about `seconds` have passed; returns (sequences, tokens, seconds)."""
    nseq, toks = 0, 0
    t0 = time.perf_counter()
    while nseq == 0 or time.perf_counter() - t0 < seconds:
        b = nseq % w.B
        O.explicit_decode(w.q_c[b], w.q_r[b], w.c_kv[b], w.k_r[b], w.w_uk, w.w_uv,
                          scale=w.scale, base=w.rope_base)
        nseq += 1
        toks += int(w.lens[b])
    return nseq, toks, time.perf_counter() - t0


def _tiny_one_thread(O, reps=200):
    """The oracle on the tiny float32 workload (one 64-token sequence, 4 heads):
    projections from the hidden states, then the explicit decode; mean time."""
    import mla_inputs as W
    t = W.make("tiny_f32")
    r = t.raw
    t0 = time.perf_counter()
    for _ in range(reps):
        c_kv, k_r, q_c, q_r = O.project(r["h"], r["w_dkv"], r["w_kr"], r["w_q"], t.n_h, t.d_h, t.d_R)
        O.explicit_decode(q_c, q_r, c_kv, k_r, r["w_uk"], r["w_uv"], scale=t.scale, base=t.rope_base)
    us = (time.perf_counter() - t0) / reps * 1e6
    return {"us_per_decode": round(us, 1), "tokens": int(t.lens[0]), "n_heads": t.n_h,
            "GBps": round(int(t.lens[0]) * t.D * 4 / (us * 1e-6) / 1e9, 4)}


def cpu_baseline(w, seconds, row_bytes):
    """The float64 oracle (explicit k_C / v reconstruction) timed on host cores
    on a bounded sample of the same workload: whole sequences with all heads,
    in batch order (wrapping round), until about `seconds` have passed; then
    the same with the BLAS pool held to one thread for a quarter of that."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import mla_oracle as O
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max((int(p.get("num_threads", 1)) for p in blas), default=1)
    nseq, toks, dt = _oracle_rate(O, w, seconds)
    with threadpool_limits(limits=1, user_api="blas"):
        n1, t1, dt1 = _oracle_rate(O, w, seconds / 4)
        tiny = _tiny_one_thread(O)
    return {"value": round(toks * row_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": _cpu_model(),
            "blas": [f"{p.get('internal_api')} {p.get('version')} x{p.get('num_threads')}" for p in blas],
            "sample": f"{nseq} sequence decodes of the {w.B}-sequence batch, in batch order "
                      f"({toks} tokens, all {w.n_h} heads), {dt:.2f} s",
            "one_thread": {"value": round(t1 * row_bytes / dt1 / 1e9, 4), "unit": "GB/s",
                           "sample": f"{n1} sequence decodes ({t1} tokens), {dt1:.2f} s, BLAS held to 1 thread"},
            "one_thread_tiny_f32": tiny}


if __name__ == "__main__":
    main()
