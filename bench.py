#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole hot path over synthetic inputs:
  * a Prefill-Only request: 28 launches (one per layer) of packed causal GQA
    prefill over 15 packed sequences, lengths uniform in [64, 480] (T = 4228),
    16 query / 8 KV heads, head dim 128, each layer with its own Q/K/V;
  * a long-prompt beam search: 8 requests x 400 beams over a 480-token shared
    prompt, 5 decode steps, each = shared-prefix decode (16/8 heads, d 128,
    suffix length = step) -> two-stage top-K over bf16 logits [8, 400, 151936]
    (2W per beam, W overall) -> parent-index suffix K/V reorder.

The headline value is the prefill attention throughput in logical TFLOP/s
(4 * D * Nq * sum L(L+1)/2 per layer, FMA = 2); decode, top-K and reorder are
reported in algorithmic GB/s. Kernel times come from HIP events on the launching
stream around launches that run back to back behind a spin gate: one pair around
the 28 prefill launches of a request (the average launch is their span / 28), and
for decode, top-K and reorder one pair around K repeats of each step's launch.
Inputs are drawn on the GPU from fixed seeds.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# HBM bytes per launch, from two rocprofv3 --pmc passes over this script (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch, averaged over the kernel's dispatches). Calibration: a plain 512 MiB
# device copy (--calib-copy-mb 512) reads FETCH_SIZE = 262156 KiB and WRITE_SIZE = 524288 KiB, so
# fetch counts are scaled by 2 and write counts by 1 (beam_topk: both of its kernels). Each figure is tied to the sources of the
# kernel it was measured on and is reported as null once they change.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
KERNEL_SOURCES = {
    "packed_gqa_prefill": ["prefill.hip", "attn_core.hpp", "device_common.hpp", "internal.hpp"],
    "shared_prefix_decode": ["decode.hip", "attn_core.hpp", "device_common.hpp", "internal.hpp"],
    "beam_topk": ["topk.hip", "device_common.hpp", "internal.hpp"],
    "suffix_reorder": ["reorder.hip", "internal.hpp"],
}
MEASURED_TRAFFIC = {
    "packed_gqa_prefill": {"fetch_kib": 17173.9, "write_kib": 17972.2, "sources_sha256": "63a7f5e4487d387a"},
    "shared_prefix_decode": {"fetch_kib": 34130.2, "write_kib": 14944.1, "sources_sha256": "35756fe22eeed70b"},
    "beam_topk": {"fetch_kib": 487023.4, "write_kib": 20037.5, "sources_sha256": "387ba3c5334eb011"},
    "suffix_reorder": {"fetch_kib": 14882.8, "write_kib": 38400.0, "sources_sha256": "8c1e96f48115f389"},
}


def sources_sha(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ["../build.py"]:
        with open(os.path.join(ROOT, "attention_bga_packed_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """Counter-derived HBM bytes per launch, or None if not measured on the current sources."""
    t = MEASURED_TRAFFIC.get(kernel)
    if t is None or t["sources_sha256"] != sources_sha(kernel):
        return None
    return int(round(t["fetch_kib"] * 1024 * FETCH_SCALE + t["write_kib"] * 1024 * WRITE_SCALE))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time budget for the oracle baseline sample (0 disables it)")
    ap.add_argument("--only", choices=["long_prefill", "long_prefill_1024", "short_decode"], default=None,
                    help="instead of the step, time one other configuration by itself (its kernel launched back "
                         "to back) and print a JSON line for it")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB (a known-size dispatch "
                         "for calibrating the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the hot path is measured on a single MI355X and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import attention_bga_packed_amd as bga
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy_mb > 0:   # one plain device copy of known size, for counter calibration
        src = torch.empty(args.calib_copy_mb << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only:
        print(json.dumps(only_config(args, dev)), flush=True)
        return

    # ---------------- inputs (resident in HBM before timing)
    pcfg = wl.CONFIGS["prefill_only"]
    lengths = wl.prefill_lengths(pcfg)
    layers = pcfg["layers"]
    cases = [wl.make_prefill_case(lengths, pcfg["nq"], pcfg["nkv"], pcfg["d"], pcfg["seed"] * 1000 + i, dev)
             for i in range(layers)]
    cu = torch.from_numpy(cases[0].cu_seqlens).to(dev)
    max_len = max(lengths)
    p_out = torch.empty_like(cases[0].q)
    p_lse = torch.empty(cases[0].q.shape[:2], dtype=torch.float32, device=dev)

    bcfg = wl.CONFIGS["long_beam"]
    R, W, LP, NS, NQ, NKV, D, V = (bcfg[k] for k in ("r", "w", "lp", "steps", "nq", "nkv", "d", "vocab"))
    dc = wl.make_named_decode("long_beam", device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(bcfg["seed"] * 7919)
    qs = [wl.bf16_normal((R, W, NQ, D), gen, dev) for _ in range(NS)]
    logits = [wl.make_logits(R, W, V, bcfg["logit_std"], bcfg["seed"] + s + 1, dev) for s in range(NS)]
    suf = [(dc.suffix_k, dc.suffix_v), (torch.empty_like(dc.suffix_k), torch.empty_like(dc.suffix_v))]
    d_out = torch.empty_like(qs[0])
    d_lse = torch.empty((R, W, NQ), dtype=torch.float32, device=dev)
    ws = torch.empty(bga.beam_topk_workspace_size(R, W, V, 2 * W, W), dtype=torch.uint8, device=dev)
    topk_out = {"tokens": torch.empty((R, W), dtype=torch.int32, device=dev),
                "parents": torch.empty((R, W), dtype=torch.int32, device=dev),
                "scores": torch.empty((R, W), dtype=torch.float32, device=dev)}
    cum = torch.zeros((R, W), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))]

    def beam_launches(s, cur):
        """The three launches of beam-search step s (suffix length s + 1), suffix buffers suf[cur] -> suf[1 - cur]."""
        sk, sv = suf[cur]
        nk, nv = suf[1 - cur]
        return (
            lambda: bga.shared_prefix_decode(qs[s], dc.prefix_k, dc.prefix_v, sk, sv, s + 1, out=d_out, lse=d_lse),
            lambda: bga.beam_topk(logits[s], cum, 2 * W, W, workspace=ws, out=topk_out),
            lambda: bga.suffix_reorder(sk, sv, topk_out["parents"], s + 1, dst_k=nk, dst_v=nv),
        )

    def step(timed):
        """One pass of the hot path; with `timed`, one HIP event pair brackets the prefill layers."""
        # the 28 layers run back to back, as in a request; one event pair spans them
        if timed:
            evs[0][0].record(stream)
        for c in cases:
            bga.packed_gqa_prefill(c.q, c.k, c.v, cu, max_len, out=p_out, lse=p_lse)
        if timed:
            evs[0][1].record(stream)
        cur = 0
        cum.zero_()
        for s in range(NS):
            for fn in beam_launches(s, cur):
                fn()
            cum.copy_(topk_out["scores"])
            cur = 1 - cur

    for _ in range(args.warmup):
        step(True)
    torch.cuda.synchronize()

    # ---- timed region: K whole steps, wall clock
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # ---- per-kernel durations: the same K steps again, HIP events on the launching stream. A spin
    # kernel queued first holds the GPU while the host enqueues the whole step, so the launches run
    # back to back and the event pairs span only the kernels (otherwise the host's per-launch
    # overhead, which exceeds a prefill launch, would be counted too).
    host_t = time.perf_counter()
    step(True)
    host_t = time.perf_counter() - host_t
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    torch.cuda._sleep(1 << 20)
    c1.record(stream)
    torch.cuda.synchronize()
    cycles_per_ms = (1 << 20) / max(c0.elapsed_time(c1), 1e-3)
    gate = int(cycles_per_ms * max(3.0 * host_t * 1e3, 2.0))

    t_pre = 0.0
    for _ in range(args.steps):
        torch.cuda._sleep(gate)
        step(True)
        torch.cuda.synchronize()   # events of this step are complete; read them
        t_pre += evs[0][0].elapsed_time(evs[0][1])

    # Beam-search kernels, each timed by itself: K launches back to back behind the gate with one event
    # pair around them (an event pair around one short launch would also count its dispatch gap), the
    # launches rotating over input sets that together exceed the 256 MB Infinity Cache (four decode
    # sets of 160 MB; the five 194 MB logits tensors). Average launch = span / K.
    dsets = [dc] + [wl.make_decode_case(R, W, LP, NS, NQ, NKV, D, bcfg["seed"] * 1000 + i, dev) for i in range(1, 4)]
    torch.cuda.synchronize()

    def back_to_back(fns):
        fns[0]()
        torch.cuda.synchronize()
        torch.cuda._sleep(gate)
        evs[0][0].record(stream)
        for i in range(args.steps):
            fns[i % len(fns)]()
        evs[0][1].record(stream)
        torch.cuda.synchronize()
        return evs[0][0].elapsed_time(evs[0][1])

    t_dec, t_reo = [0.0] * NS, [0.0] * NS
    for s in range(NS):
        t_dec[s] = back_to_back([lambda ds=ds, s=s: bga.shared_prefix_decode(ds.q, ds.prefix_k, ds.prefix_v, ds.suffix_k,
                                                                              ds.suffix_v, s + 1, out=d_out, lse=d_lse)
                                 for ds in dsets])
        t_reo[s] = back_to_back([lambda ds=ds, s=s: bga.suffix_reorder(ds.suffix_k, ds.suffix_v, topk_out["parents"],
                                                                        s + 1, dst_k=suf[1][0], dst_v=suf[1][1])
                                 for ds in dsets])
    t_top = [back_to_back([lambda j=j: bga.beam_topk(logits[j], cum, 2 * W, W, workspace=ws, out=topk_out)
                           for j in range(NS)])] * NS

    K = args.steps
    pre_flops = wl.prefill_flops(lengths, pcfg["nq"], pcfg["d"])
    pre_ms = t_pre / (K * layers)                           # average launch, ms
    pre_tflops = pre_flops / (pre_ms * 1e-3) / 1e12
    dec_bytes = [wl.decode_bytes(R, W, NQ, NKV, LP, s + 1, D) for s in range(NS)]
    dec_ms = [t / K for t in t_dec]
    dec_gbs = sum(dec_bytes) / (sum(dec_ms) * 1e-3) / 1e9
    dec_flops = sum(wl.decode_flops(R, W, NQ, LP, s + 1, D) for s in range(NS))
    top_bytes = wl.topk_bytes(R, W, V, W)
    top_ms = sum(t_top) / (K * NS)
    top_gbs = top_bytes / (top_ms * 1e-3) / 1e9
    reo_bytes = [wl.reorder_bytes(R, W, s + 1, NKV, D) for s in range(NS)]
    reo_ms = [t / K for t in t_reo]
    reo_gbs = sum(reo_bytes) / (sum(reo_ms) * 1e-3) / 1e9

    def roof(kernel, bound, achieved, peak, unit, per_launch, ms):
        return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(kernel),
                "algorithmic_per_launch": per_launch, "avg_launch_us": round(ms * 1e3, 2)}

    # The prefill layer's roofline follows from its arithmetic intensity: below the ridge
    # (2500 TFLOP/s / 8000 GB/s = 312.5 FLOP/B) HBM bounds it, above it the matrix cores do.
    pre_bytes = wl.prefill_bytes(lengths, pcfg["nq"], pcfg["nkv"], pcfg["d"])
    pre_gbs = pre_bytes / (pre_ms * 1e-3) / 1e9
    if pre_flops / pre_bytes < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        pre_roof = roof("packed_gqa_prefill", "hbm", pre_gbs, PEAK_HBM_GBS, "GB/s", pre_bytes, pre_ms)
    else:
        pre_roof = roof("packed_gqa_prefill", "mfma", pre_tflops, PEAK_BF16_TFLOPS, "TFLOP/s", pre_flops, pre_ms)
    pre_roof.update({"flop_per_byte": round(pre_flops / pre_bytes, 1), "tflops": round(pre_tflops, 2),
                     "mfma_frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4), "gbs": round(pre_gbs, 1),
                     "hbm_frac": round(pre_gbs / PEAK_HBM_GBS, 4)})
    rooflines = {
        "packed_gqa_prefill": pre_roof,
        "shared_prefix_decode": roof("shared_prefix_decode", "hbm", dec_gbs, PEAK_HBM_GBS, "GB/s", int(np.mean(dec_bytes)),
                                     float(np.mean(dec_ms))),
        "beam_topk": roof("beam_topk", "hbm", top_gbs, PEAK_HBM_GBS, "GB/s", top_bytes, top_ms),
        "suffix_reorder": roof("suffix_reorder", "hbm", reo_gbs, PEAK_HBM_GBS, "GB/s", int(np.mean(reo_bytes)),
                               float(np.mean(reo_ms))),
    }
    rooflines["shared_prefix_decode"]["mfma_tflops"] = round(dec_flops / (sum(dec_ms) * 1e-3) / 1e12, 2)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(cases[0], pre_flops, args.cpu_seconds)

    rec = {
        "metric": "attention TFLOPS & %bf16 MFMA peak (prefill); GB/s & %HBM peak (beam decode)",
        "value": round(pre_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, N(0,3) logits; no weights)",
        "config": {
            "workload": "prefill_only x28 layers + long_beam 5-step beam search",
            "prefill": {"sequences": len(lengths), "total_tokens": int(sum(lengths)), "max_len": max_len,
                        "num_q_heads": pcfg["nq"], "num_kv_heads": pcfg["nkv"], "head_dim": pcfg["d"],
                        "launches_per_step": layers},
            "beam": {"requests": R, "beams": W, "prefix_len": LP, "decode_steps": NS, "num_q_heads": NQ,
                     "num_kv_heads": NKV, "head_dim": D, "vocab": V, "k_local": 2 * W, "k_global": W},
            "global_batch": len(lengths),
            "seq_len": max_len,
        },
        "prefill_pct_bf16_peak": round(100 * pre_tflops / PEAK_BF16_TFLOPS, 2),
        "decode_gbs": round(dec_gbs, 1),
        "decode_pct_hbm_peak": round(100 * dec_gbs / PEAK_HBM_GBS, 2),
        "decode_us_per_step": [round(t * 1e3, 2) for t in dec_ms],
        "topk_gbs": round(top_gbs, 1),
        "reorder_gbs": round(reo_gbs, 1),
        "roofline": rooflines["packed_gqa_prefill"],
        "rooflines": rooflines,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def timed_launches(fn, n, warmup):
    """Average duration (ms) of n back-to-back calls fn(i), measured with HIP events on the launching stream
    behind a spin gate (so the host's launch overhead is not counted)."""
    import torch
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        fn(i)
    torch.cuda.synchronize()
    host = time.perf_counter() - t0
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    torch.cuda._sleep(1 << 20)
    b.record(stream)
    torch.cuda.synchronize()
    gate = int((1 << 20) / max(a.elapsed_time(b), 1e-3) * max(3.0 * host * 1e3, 2.0))
    torch.cuda._sleep(gate)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def only_config(args, dev):
    """One configuration other than the step's, timed by itself (--only)."""
    import torch

    import attention_bga_packed_amd as bga
    import workloads as wl

    name, K, W0 = args.only, max(args.steps, 1), max(args.warmup, 1)
    cfg = wl.CONFIGS[name]
    rec = {"metric": "attention TFLOPS & %bf16 MFMA peak (prefill); GB/s & %HBM peak (beam decode)",
           "n_gpus": 1, "steps": K, "warmup": W0, "higher_is_better": True, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) Q/K/V)", "vs_baseline": None}
    if cfg["kind"] == "prefill":
        lengths = wl.prefill_lengths(cfg)
        # input sets rotated between launches: together larger than the 256 MB Infinity Cache
        nsets = 2 if name == "long_prefill_1024" else 3
        cases = [wl.make_prefill_case(lengths, cfg["nq"], cfg["nkv"], cfg["d"], cfg["seed"] * 1000 + i, dev)
                 for i in range(nsets)]
        cu = torch.from_numpy(cases[0].cu_seqlens).to(dev)
        out = torch.empty_like(cases[0].q)
        lse = torch.empty(cases[0].q.shape[:2], dtype=torch.float32, device=dev)
        ms = timed_launches(lambda i: bga.packed_gqa_prefill(cases[i % nsets].q, cases[i % nsets].k, cases[i % nsets].v,
                                                             cu, max(lengths), out=out, lse=lse), K, W0)
        flops = wl.prefill_flops(lengths, cfg["nq"], cfg["d"])
        t = sum(lengths)
        hbm = wl.prefill_bytes(lengths, cfg["nq"], cfg["nkv"], cfg["d"])
        tf = flops / (ms * 1e-3) / 1e12
        gbs = hbm / (ms * 1e-3) / 1e9
        if flops / hbm < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
            roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_per_launch": hbm}
        else:
            roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / PEAK_BF16_TFLOPS, 4), "algorithmic_per_launch": flops}
        roof.update({"traffic": None, "avg_launch_us": round(ms * 1e3, 2), "flop_per_byte": round(flops / hbm, 1),
                     "tflops": round(tf, 2), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4), "gbs": round(gbs, 1),
                     "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)})
        rec.update({"value": round(tf, 3), "unit": "TFLOP/s", "ms_per_step": round(ms, 4),
                    "config": {"workload": name, "sequences": len(lengths), "total_tokens": t,
                               "max_len": max(lengths), "num_q_heads": cfg["nq"], "num_kv_heads": cfg["nkv"],
                               "head_dim": cfg["d"], "input_sets": nsets},
                    "roofline": roof})
        return rec
    # decode: every suffix length of the configuration, several input sets rotated
    nsets = 4
    cases = [wl.make_decode_case(cfg["r"], cfg["w"], cfg["lp"], cfg["ls_cap"], cfg["nq"], cfg["nkv"], cfg["d"],
                                 cfg["seed"] * 1000 + i, dev) for i in range(nsets)]
    out = torch.empty_like(cases[0].q)
    lse = torch.empty(cases[0].q.shape[:3], dtype=torch.float32, device=dev)
    per, tot_b, tot_ms = [], 0, 0.0
    for ls in range(1, cfg["steps"] + 1):
        ms = timed_launches(lambda i: bga.shared_prefix_decode(cases[i % nsets].q, cases[i % nsets].prefix_k,
                                                               cases[i % nsets].prefix_v, cases[i % nsets].suffix_k,
                                                               cases[i % nsets].suffix_v, ls, out=out, lse=lse), K, W0)
        b = wl.decode_bytes(cfg["r"], cfg["w"], cfg["nq"], cfg["nkv"], cfg["lp"], ls, cfg["d"])
        per.append(round(ms * 1e3, 2))
        tot_b += b
        tot_ms += ms
    gbs = tot_b / (tot_ms * 1e-3) / 1e9
    rec.update({"value": round(gbs, 1), "unit": "GB/s", "ms_per_step": round(tot_ms / cfg["steps"], 4),
                "decode_us_per_step": per,
                "config": {"workload": name, "requests": cfg["r"], "beams": cfg["w"], "prefix_len": cfg["lp"],
                           "decode_steps": cfg["steps"], "num_q_heads": cfg["nq"], "num_kv_heads": cfg["nkv"],
                           "head_dim": cfg["d"], "input_sets": nsets},
                "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                             "algorithmic_per_launch": tot_b // cfg["steps"],
                             "avg_launch_us": round(tot_ms / cfg["steps"] * 1e3, 2)}})
    return rec


def cpu_baseline(case, flops, seconds):
    """The fp64 oracle on one Prefill-Only layer, repeated until ~`seconds` of CPU work."""
    import oracle
    import numpy as np

    q, k, v = case.q.cpu(), case.k.cpu(), case.v.cpu()
    cu = np.asarray(case.cu_seqlens)
    threads = oracle.num_threads(0)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.packed_prefill(q, k, v, cu, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    return {"value": round(flops * reps / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x one Prefill-Only layer (15 sequences, T={int(cu[-1])}, 16/8 heads, d 128) "
                      f"in {el:.1f} s"}


if __name__ == "__main__":
    main()
