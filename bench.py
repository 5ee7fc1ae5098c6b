#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input of
every measured workload:
  * Prefill-Only request: 28 launches (one per layer, each with its own Q/K/V)
    of packed causal GQA prefill over 15 sequences, lengths uniform in
    [64, 480] (T = 4228), 16 query / 8 KV heads, head dim 128;
  * long packed prefill: 120 sequences, lognormal lengths (median 400,
    sigma 0.4, clipped to [32, 1024]; T = 52,348), 14 / 2 heads, head dim 64;
  * long packed prefill, 120 x 1024 tokens (T = 122,880), 14 / 2 heads, d 64;
  * short-prompt beam decode: 32 requests x 100 beams over a 128-token shared
    prompt, 4 steps of shared-prefix decode (16 / 8 heads, d 64, suffix length
    = step) + parent-index suffix reorder (parents drawn uniformly);
  * long-prompt beam search: 8 requests x 400 beams over a 480-token prompt,
    5 steps of shared-prefix decode (16 / 8 heads, d 128) -> two-stage top-K
    over bf16 logits [8, 400, 151936] (2W per beam, W overall) -> reorder.

The headline value is the prefill attention throughput on the 120 x 1024 batch,
the one prefill workload whose arithmetic intensity (442 FLOP/B) is above the
MI355X ridge (2500 TFLOP/s / 8 TB/s = 312.5 FLOP/B), in logical TFLOP/s
(4 * D * Nq * sum L(L+1)/2, FMA = 2), with its roofline against the bf16 MFMA
peak. `rooflines` holds every kernel and workload: prefill in TFLOP/s and
algorithmic GB/s (bound by the intensity), decode, top-K and reorder in
algorithmic GB/s. Kernel durations come from HIP events on the launching
stream around launches that run back to back behind a spin gate, rotating over
input sets that together exceed the 256 MB Infinity Cache. `cpu_baseline`
times the fp64 oracle on the headline workload on the host cores (median of
three); `cpu_baselines` does the same for every operation on bounded samples.
Inputs are drawn on the GPU from fixed seeds and are resident in HBM before
any timing. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # FLOP/B
METRIC = "attention TFLOPS & %bf16 MFMA peak (prefill); GB/s & %HBM peak (beam decode)"

# HBM bytes per launch, from two rocprofv3 --pmc passes over this script (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch, averaged over the workload's dispatches). Calibration: a plain
# 512 MiB device copy (--calib-copy-mb 512) reads FETCH_SIZE = 262156 KiB and WRITE_SIZE =
# 524288 KiB, so fetch counts are scaled by 2 and write counts by 1. Each figure is tied to a
# hash of the sources of the kernel it was measured on and is reported as null once they change.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
KERNEL_SOURCES = {
    "packed_gqa_prefill": ["prefill.hip", "attn_core.hpp", "device_common.hpp", "internal.hpp"],
    "shared_prefix_decode": ["decode.hip", "attn_core.hpp", "device_common.hpp", "internal.hpp"],
    "beam_topk": ["topk.hip", "device_common.hpp", "internal.hpp"],
    "suffix_reorder": ["reorder.hip", "internal.hpp"],
    "swiglu_quant": ["swiglu_fp8.hip", "device_common.hpp", "internal.hpp"],
}
# workload -> {"kernel", "fetch_kib", "write_kib", "sources_sha256"}
# (measured with the command lines in profiles/hbm_counters_by_workload.md)
MEASURED_TRAFFIC: dict = {
    "prefill_only": {"kernel": "packed_gqa_prefill", "fetch_kib": 17135.2, "write_kib": 17972.3, "sources_sha256": "e9abfae5b6580973"},
    "long_prefill": {"kernel": "packed_gqa_prefill", "fetch_kib": 62363.0, "write_kib": 112737.9, "sources_sha256": "e9abfae5b6580973"},
    "long_prefill_1024": {"kernel": "packed_gqa_prefill", "fetch_kib": 139672.7, "write_kib": 252321.0, "sources_sha256": "e9abfae5b6580973"},
    "short_decode/decode": {"kernel": "shared_prefix_decode", "fetch_kib": 15425.6, "write_kib": 7200.0, "sources_sha256": "6f5b3400c5b60814"},
    "short_decode/reorder": {"kernel": "suffix_reorder", "fetch_kib": 7693.0, "write_kib": 16024.9, "sources_sha256": "e0ef6d4301e3490d"},
    "long_beam/decode": {"kernel": "shared_prefix_decode", "fetch_kib": 34381.4, "write_kib": 15392.0, "sources_sha256": "6f5b3400c5b60814"},
    "long_beam/reorder": {"kernel": "suffix_reorder", "fetch_kib": 14329.8, "write_kib": 38460.5, "sources_sha256": "e0ef6d4301e3490d"},
    "long_beam/topk": {"kernel": "beam_topk", "fetch_kib": 475894.7, "write_kib": 20037.5, "sources_sha256": "5d5c523849b895fa"},
    "swiglu_fp8": {"kernel": "swiglu_quant", "fetch_kib": 33840.5, "write_kib": 17044.1, "sources_sha256": "58bd510a4b1ecb4f"},
}


def sources_sha(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ["../build.py"]:
        with open(os.path.join(ROOT, "attention_bga_packed_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """Counter-derived HBM bytes per launch, or None if not measured on the current sources."""
    t = MEASURED_TRAFFIC.get(workload)
    if t is None or t["sources_sha256"] != sources_sha(t["kernel"]):
        return None
    return int(round(t["fetch_kib"] * 1024 * FETCH_SCALE + t["write_kib"] * 1024 * WRITE_SCALE))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=1.0,
                    help="scale of the oracle baselines (0 disables them; 1 = the default samples, ~15 s)")
    ap.add_argument("--only", choices=["prefill_only", "long_prefill", "long_prefill_1024", "short_decode",
                                       "long_beam", "swiglu_fp8", "long_beam_loop"], default=None,
                    help="run (and time) only this workload's launches; for profiling one workload")
    ap.add_argument("--no-comparators", action="store_true",
                    help="skip the Torch baselines of the article's relative claims")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB (a known-size dispatch "
                         "for calibrating the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


class Timer:
    """Average duration of back-to-back launches: HIP events on the launching stream around n calls,
    queued behind a spin kernel that holds the GPU while the host enqueues them (so the host's
    per-launch overhead is not counted)."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        torch.cuda._sleep(1 << 20)
        b.record(self.stream)
        torch.cuda.synchronize()
        self.cycles_per_ms = (1 << 20) / max(a.elapsed_time(b), 1e-3)

    def span_ms(self, fns, n):
        """Total ms of n back-to-back calls cycling over fns (host enqueue hidden behind a gate)."""
        torch = self.torch
        fns[0]()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            fns[i % len(fns)]()
        torch.cuda.synchronize()
        host_ms = (time.perf_counter() - t0) * 1e3
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(self.cycles_per_ms * max(3.0 * host_ms, 2.0)))
        a.record(self.stream)
        for i in range(n):
            fns[i % len(fns)]()
        b.record(self.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def per_launch_us(self, fns, n):
        """p10 / p50 / p90 of single launches (µs): n back-to-back calls cycling over fns behind the
        same gate, an event recorded between consecutive calls."""
        torch = self.torch
        fns[0]()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        t0 = time.perf_counter()
        for i in range(n):
            fns[i % len(fns)]()
        torch.cuda.synchronize()
        host_ms = (time.perf_counter() - t0) * 1e3
        torch.cuda._sleep(int(self.cycles_per_ms * max(3.0 * host_ms, 2.0)))
        evs[0].record(self.stream)
        for i in range(n):
            fns[i % len(fns)]()
            evs[i + 1].record(self.stream)
        torch.cuda.synchronize()
        d = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n))
        pick = lambda q: round(d[min(n - 1, int(q * (n - 1) + 0.5))], 2)
        return {"launch_us_p10": pick(0.1), "launch_us_p50": pick(0.5), "launch_us_p90": pick(0.9), "launches": n}


def build_inputs(dev, only=None):
    """Every workload's inputs and launch closures, resident in HBM. Returns {workload: dict}."""
    W = {}
    for name, make in (("prefill_only", lambda: prefill_workload("prefill_only", None, dev)),
                       ("long_prefill", lambda: prefill_workload("long_prefill", 3, dev)),
                       ("long_prefill_1024", lambda: prefill_workload("long_prefill_1024", 2, dev)),
                       ("short_decode", lambda: short_decode_workload(dev)),
                       ("long_beam", lambda: long_beam_workload(dev)),
                       ("swiglu_fp8", lambda: swiglu_workload(dev)),
                       ("long_beam_loop", lambda: beam_loop_workload(dev))):
        if only is None or only == name:
            W[name] = make()
    return W


def prefill_workload(name, nsets, dev):
    """One input set per launch of a step (Prefill-Only: one per layer); the long batches have several
    sets, rotated when timed so that together they exceed the Infinity Cache."""
    import torch

    import attention_bga_packed_amd as bga
    import workloads as wl

    cfg = wl.CONFIGS[name]
    lengths = wl.prefill_lengths(cfg)
    n = cfg.get("layers", nsets)
    cases = [wl.make_prefill_case(lengths, cfg["nq"], cfg["nkv"], cfg["d"], cfg["seed"] * 1000 + i, dev)
             for i in range(n)]
    cu = torch.from_numpy(cases[0].cu_seqlens).to(dev)
    out = torch.empty_like(cases[0].q)
    lse = torch.empty(cases[0].q.shape[:2], dtype=torch.float32, device=dev)
    mx = max(lengths)
    fns = [lambda c=c: bga.packed_gqa_prefill(c.q, c.k, c.v, cu, mx, out=out, lse=lse) for c in cases]
    w = dict(kind="prefill", cfg=cfg, lengths=lengths, cases=cases, fns=fns,
             step_launches=fns if name == "prefill_only" else fns[:1])
    if name == "prefill_only":
        # the request's output rows at each sequence's last token (the input of the per-sample head)
        last = torch.empty((len(lengths),) + tuple(out.shape[1:]), dtype=out.dtype, device=dev)
        w["gather"] = lambda: bga.last_token_gather(out, cu, out=last)
        w["step_launches"] = fns + [w["gather"]]
    return w


def short_decode_workload(dev):
    """4 steps of shared-prefix decode + reorder with parents drawn uniformly (no top-K in this workload)."""
    import torch

    import attention_bga_packed_amd as bga
    import workloads as wl

    cfg = wl.CONFIGS["short_decode"]
    R, Wb, LP, NS = cfg["r"], cfg["w"], cfg["lp"], cfg["steps"]
    sets = [wl.make_decode_case(R, Wb, LP, cfg["ls_cap"], cfg["nq"], cfg["nkv"], cfg["d"], cfg["seed"] * 1000 + i,
                                dev) for i in range(4)]
    parents = [torch.from_numpy(wl.make_parents(R, Wb, Wb, cfg["seed"] + 10 * s)).to(dev) for s in range(NS)]
    out = torch.empty_like(sets[0].q)
    lse = torch.empty(sets[0].q.shape[:3], dtype=torch.float32, device=dev)
    bufs = [(sets[0].suffix_k, sets[0].suffix_v), (torch.empty_like(sets[0].suffix_k),
                                                     torch.empty_like(sets[0].suffix_v))]

    def step():
        cur = 0
        for s in range(NS):
            sk, sv = bufs[cur]
            bga.shared_prefix_decode(sets[0].q, sets[0].prefix_k, sets[0].prefix_v, sk, sv, s + 1, out=out, lse=lse)
            bga.suffix_reorder(sk, sv, parents[s], s + 1, dst_k=bufs[1 - cur][0], dst_v=bufs[1 - cur][1])
            cur = 1 - cur

    dec = [[lambda c=c, s=s: bga.shared_prefix_decode(c.q, c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v, s + 1,
                                                      out=out, lse=lse) for c in sets] for s in range(NS)]
    reo = [[lambda c=c, s=s: bga.suffix_reorder(c.suffix_k, c.suffix_v, parents[s], s + 1, dst_k=bufs[1][0],
                                                dst_v=bufs[1][1]) for c in sets] for s in range(NS)]
    return dict(kind="beam", cfg=cfg, sets=sets, parents=parents, step=step, decode=dec, reorder=reo)


def long_beam_workload(dev):
    """5 steps of shared-prefix decode -> two-stage top-K -> reorder by the selected parents."""
    import torch

    import attention_bga_packed_amd as bga
    import workloads as wl

    cfg = wl.CONFIGS["long_beam"]
    R, Wb, LP, NS, NQ, NKV, D, V = (cfg[k] for k in ("r", "w", "lp", "steps", "nq", "nkv", "d", "vocab"))
    sets = [wl.make_named_decode("long_beam", device=dev)] + [
        wl.make_decode_case(R, Wb, LP, NS, NQ, NKV, D, cfg["seed"] * 1000 + i, dev) for i in range(1, 4)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg["seed"] * 7919)
    qs = [wl.bf16_normal((R, Wb, NQ, D), gen, dev) for _ in range(NS)]
    logits = [wl.make_logits(R, Wb, V, cfg["logit_std"], cfg["seed"] + s + 1, dev) for s in range(NS)]
    dc = sets[0]
    bufs = [(dc.suffix_k, dc.suffix_v), (torch.empty_like(dc.suffix_k), torch.empty_like(dc.suffix_v))]
    out = torch.empty_like(qs[0])
    lse = torch.empty((R, Wb, NQ), dtype=torch.float32, device=dev)
    ws = torch.empty(bga.beam_topk_workspace_size(R, Wb, V, 2 * Wb, Wb), dtype=torch.uint8, device=dev)
    tk = {"tokens": torch.empty((R, Wb), dtype=torch.int32, device=dev),
          "parents": torch.empty((R, Wb), dtype=torch.int32, device=dev),
          "scores": torch.empty((R, Wb), dtype=torch.float32, device=dev)}
    cum = torch.zeros((R, Wb), dtype=torch.float32, device=dev)

    def step():
        cur = 0
        cum.zero_()
        for s in range(NS):
            sk, sv = bufs[cur]
            nk, nv = bufs[1 - cur]
            bga.shared_prefix_decode(qs[s], dc.prefix_k, dc.prefix_v, sk, sv, s + 1, out=out, lse=lse)
            bga.beam_topk(logits[s], cum, 2 * Wb, Wb, workspace=ws, out=tk)
            bga.suffix_reorder(sk, sv, tk["parents"], s + 1, dst_k=nk, dst_v=nv)
            cum.copy_(tk["scores"])
            cur = 1 - cur

    dec = [[lambda c=c, s=s: bga.shared_prefix_decode(c.q, c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v, s + 1,
                                                      out=out, lse=lse) for c in sets] for s in range(NS)]
    reo = [[lambda c=c, s=s: bga.suffix_reorder(c.suffix_k, c.suffix_v, tk["parents"], s + 1, dst_k=bufs[1][0],
                                                dst_v=bufs[1][1]) for c in sets] for s in range(NS)]
    top = [lambda j=j: bga.beam_topk(logits[j], cum, 2 * Wb, Wb, workspace=ws, out=tk) for j in range(NS)]
    return dict(kind="beam", cfg=cfg, sets=sets, step=step, decode=dec, reorder=reo, topk=top, logits=logits)


def swiglu_workload(dev):
    """The fused SwiGLU + E4M3 requantisation over the Prefill-Only request's tokens; five input sets (87 MB of
    traffic each) rotated when timed."""
    import torch

    import attention_bga_packed_amd as bga
    import workloads as wl

    cfg = wl.CONFIGS["swiglu_fp8"]
    t, i = cfg["tokens"], cfg["inter"]
    sets = []
    for k in range(5):
        g = torch.Generator(device=dev)
        g.manual_seed(cfg["seed"] * 1000 + k)
        sets.append(wl.bf16_normal((t, 2 * i), g, dev, cfg["std"]))
    codes = torch.empty((t, i), dtype=torch.uint8, device=dev)
    scale = torch.empty((t,), dtype=torch.float32, device=dev)
    fns = [lambda x=x: bga.swiglu_quant_e4m3(x, codes=codes, scale=scale) for x in sets]
    return dict(kind="swiglu", cfg=cfg, fns=fns, step_launches=fns[:1])


def beam_loop_workload(dev):
    """The whole fixed-depth beam search of the long-prompt configuration (8 requests x 400 beams, 480-token
    prompts, vocabulary 151936): first-step selection, then 5 steps of [suffix append -> shared-prefix decode
    -> top-K (2W / 2W) -> stop-token split -> reorder], then the final ranking. The model's outputs (query, the
    current token's K/V, logits N(0, 3)) are synthetic and resident; token 2 stops a hypothesis."""
    import torch

    import workloads as wl
    from attention_bga_packed_amd.beam_search import BeamSearch

    cfg = wl.CONFIGS["long_beam"]
    R, Wb, LP, NS, NQ, NKV, D, V = (cfg[k] for k in ("r", "w", "lp", "steps", "nq", "nkv", "d", "vocab"))
    n_gen = NS + 1
    g = torch.Generator(device=dev)
    g.manual_seed(cfg["seed"] * 31)
    pk = wl.bf16_normal((R * LP, NKV, D), g, dev)
    pv = wl.bf16_normal((R * LP, NKV, D), g, dev)
    pcu = torch.arange(0, (R + 1) * LP, LP, dtype=torch.int32, device=dev)
    model = {0: {"logits": wl.bf16_normal((R, 1, V), g, dev, cfg["logit_std"])}}
    for s in range(1, n_gen):
        model[s] = {"q": wl.bf16_normal((R, Wb, NQ, D), g, dev), "k": wl.bf16_normal((R, Wb, NKV, D), g, dev),
                    "v": wl.bf16_normal((R, Wb, NKV, D), g, dev),
                    "logits": wl.bf16_normal((R, Wb, V), g, dev, cfg["logit_std"])}
    bs = BeamSearch(R, Wb, n_gen, V, NQ, NKV, D, 2, dev)

    def loop():
        bs.start(pk, pv, pcu, model[0]["logits"])
        for s in range(1, n_gen):
            m = model[s]
            bs.decode(m["q"], m["k"], m["v"])
            bs.select(m["logits"])
        bs.finish()

    # algorithmic bytes of one loop: the kernels' own counts summed
    b = wl.topk_bytes(R, 1, V, 2 * Wb) + wl.beam_advance_bytes(R, Wb, 1, 0)
    for s in range(1, n_gen):
        b += wl.suffix_append_bytes(R, Wb, NKV, D) + wl.decode_bytes(R, Wb, NQ, NKV, LP, s, D)
        b += wl.topk_bytes(R, Wb, V, 2 * Wb) + wl.beam_advance_bytes(R, Wb, Wb, s)
        b += wl.reorder_bytes(R, Wb, s, NKV, D)
    return dict(kind="loop", cfg=cfg, fns=[loop], step_launches=[loop], bytes=b, n_gen=n_gen, bs=bs)


def roof(bound, achieved, peak, unit, per_launch, ms, traffic):
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic, "algorithmic_per_launch": per_launch,
            "avg_launch_us": round(ms * 1e3, 2)}


def prefill_roofline(name, w, ms):
    import workloads as wl
    cfg, lengths = w["cfg"], w["lengths"]
    flops = wl.prefill_flops(lengths, cfg["nq"], cfg["d"])
    hbm = wl.prefill_bytes(lengths, cfg["nq"], cfg["nkv"], cfg["d"])
    tf = flops / (ms * 1e-3) / 1e12
    gbs = hbm / (ms * 1e-3) / 1e9
    traffic = measured_traffic(name)
    if flops / hbm >= RIDGE:
        r = roof("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s", flops, ms, traffic)
    else:
        r = roof("hbm", gbs, PEAK_HBM_GBS, "GB/s", hbm, ms, traffic)
    r.update({"kernel": "packed_prefill_kernel", "flop_per_byte": round(flops / hbm, 1), "tflops": round(tf, 2),
              "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4), "gbs": round(gbs, 1),
              "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_flops": flops, "algorithmic_bytes": hbm})
    return r


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the hot path is measured on a single MI355X and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

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

    W = build_inputs(dev, args.only)
    torch.cuda.synchronize()

    def step():
        for name in ("prefill_only", "long_prefill", "long_prefill_1024", "swiglu_fp8", "long_beam_loop"):
            if name in W:
                for fn in W[name]["step_launches"]:
                    fn()
        for name in ("short_decode", "long_beam"):
            if name in W:
                W[name]["step"]()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K whole steps, wall clock
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    K = args.steps

    # ---- per-kernel durations (events around back-to-back launches, inputs rotated)
    timer = Timer(torch)
    rooflines, detail = {}, {}
    for name in ("prefill_only", "long_prefill", "long_prefill_1024"):
        if name not in W:
            continue
        w = W[name]
        n = len(w["fns"]) * max(1, K // len(w["fns"])) if name == "prefill_only" else max(K, 2 * len(w["fns"]))
        ms = timer.span_ms(w["fns"], n) / n
        rooflines[name] = prefill_roofline(name, w, ms)
        rooflines[name].update(timer.per_launch_us(w["fns"], max(n, 20)))
    if "prefill_only" in W:
        w, cfg = W["prefill_only"], W["prefill_only"]["cfg"]
        n = max(K, 8)
        ms = timer.span_ms([w["gather"]], n) / n
        b = wl.gather_bytes(len(w["lengths"]), cfg["nq"] * cfg["d"] * 2)
        r = roof("hbm", b / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s", b, ms, None)
        r.update({"kernel": "last_token_gather_kernel", "note": "15 rows of 4 KB: bound by launch latency"})
        rooflines["prefill_only/last_token_gather"] = r
    if "swiglu_fp8" in W:
        w, cfg = W["swiglu_fp8"], W["swiglu_fp8"]["cfg"]
        n = max(K, 2 * len(w["fns"]))
        ms = timer.span_ms(w["fns"], n) / n
        b = wl.swiglu_quant_bytes(cfg["tokens"], cfg["inter"])
        r = roof("hbm", b / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s", b, ms, measured_traffic("swiglu_fp8"))
        r.update({"kernel": "swiglu_quant_kernel"})
        r.update(timer.per_launch_us(w["fns"], max(n, 20)))
        rooflines["swiglu_fp8"] = r
    if "long_beam_loop" in W:
        w = W["long_beam_loop"]
        n = max(3, K // 3)
        ms = timer.span_ms(w["fns"], n) / n
        r = roof("hbm", w["bytes"] / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s", w["bytes"], ms, None)
        r.update({"kernel": "the whole loop (append, decode, top-K, advance, reorder, finalize)",
                  "ms_per_loop": round(ms, 4), "generated_tokens": w["n_gen"],
                  "finished_per_request": [int(x) for x in w["bs"].pool["count"].cpu()]})
        rooflines["long_beam_loop"] = r
    for name in ("short_decode", "long_beam"):
        if name not in W:
            continue
        w, cfg = W[name], W[name]["cfg"]
        R, Wb, NS = cfg["r"], cfg["w"], cfg["steps"]
        n = max(K, 8)
        dec_ms = [timer.span_ms(w["decode"][s], n) / n for s in range(NS)]
        reo_ms = [timer.span_ms(w["reorder"][s], n) / n for s in range(NS)]
        dec_b = [wl.decode_bytes(R, Wb, cfg["nq"], cfg["nkv"], cfg["lp"], s + 1, cfg["d"]) for s in range(NS)]
        dec_f = [wl.decode_flops(R, Wb, cfg["nq"], cfg["lp"], s + 1, cfg["d"]) for s in range(NS)]
        reo_b = [wl.reorder_bytes(R, Wb, s + 1, cfg["nkv"], cfg["d"]) for s in range(NS)]
        gbs = sum(dec_b) / (sum(dec_ms) * 1e-3) / 1e9
        r = roof("hbm", gbs, PEAK_HBM_GBS, "GB/s", int(np.mean(dec_b)), float(np.mean(dec_ms)),
                 measured_traffic(f"{name}/decode"))
        pl = [timer.per_launch_us(w["decode"][s], max(n, 10)) for s in range(NS)]
        r.update({k: [x[k] for x in pl] for k in ("launch_us_p10", "launch_us_p50", "launch_us_p90")})
        r.update({"kernel": "shared_prefix_decode_kernel", "us_per_step": [round(t * 1e3, 2) for t in dec_ms],
                  "mfma_tflops": round(sum(dec_f) / (sum(dec_ms) * 1e-3) / 1e12, 2),
                  "mfma_frac": round(sum(dec_f) / (sum(dec_ms) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
        rooflines[f"{name}/decode"] = r
        gbs = sum(reo_b) / (sum(reo_ms) * 1e-3) / 1e9
        r = roof("hbm", gbs, PEAK_HBM_GBS, "GB/s", int(np.mean(reo_b)), float(np.mean(reo_ms)),
                 measured_traffic(f"{name}/reorder"))
        pl = [timer.per_launch_us(w["reorder"][s], max(n, 10)) for s in range(NS)]
        r.update({k: [x[k] for x in pl] for k in ("launch_us_p10", "launch_us_p50", "launch_us_p90")})
        r.update({"kernel": "suffix_reorder_kernel", "us_per_step": [round(t * 1e3, 2) for t in reo_ms]})
        rooflines[f"{name}/reorder"] = r
        if "topk" in w:
            n = max(K, 2 * len(w["topk"]))
            ms = timer.span_ms(w["topk"], n) / n
            b = wl.topk_bytes(R, Wb, cfg["vocab"], Wb)
            r = roof("hbm", b / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s", b, ms, measured_traffic(f"{name}/topk"))
            r.update({"kernel": "topk_stage1_kernel + topk_stage2_kernel"})
            r.update(timer.per_launch_us(w["topk"], max(n, 10)))
            rooflines[f"{name}/topk"] = r

    headline = "long_prefill_1024" if "long_prefill_1024" in rooflines else next(iter(rooflines))
    hr = rooflines[headline]
    if "tflops" in hr:
        value, unit = hr["tflops"], "TFLOP/s"
    else:
        value, unit = hr["achieved"], hr["unit"]

    comps = None if args.no_comparators else comparator_timings(W, timer, rooflines)

    cpu = cpus = None
    if args.cpu_seconds > 0 and args.only is None:
        cpus = cpu_baselines(W, args.cpu_seconds)
        cpu = cpus.get("long_prefill_1024")

    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
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
            "workload": ("one pass over every measured workload: Prefill-Only request (28 layers + last-token "
                         "gather), long packed prefill (120 lognormal), long packed prefill 120 x 1024 (headline), "
                         "short-prompt beam decode (4 steps), long-prompt beam search (5 steps), SwiGLU E4M3 "
                         "requantisation (4228 x 4096), the long-prompt fixed-depth beam loop with the 2W stop rule"
                         ) if args.only is None else args.only,
            "headline": headline,
            "workloads": {n: workload_config(W[n]) for n in W},
            "global_batch": 120 if args.only is None else None,
            "seq_len": 1024 if args.only is None else None,
        },
        "roofline": hr,
        "rooflines": rooflines,
        "cpu_baseline": cpu,
        "cpu_baselines": cpus,
        "comparators": comps,
    }
    print(json.dumps(rec), flush=True)


def comparator_timings(W, timer, rooflines):
    """The article's relative claims restated per kernel on this GPU: explicit Torch prefill (padded; packed
    block-diagonal for the Prefill-Only request) against the packed prefill kernel, and the per-beam full K/V
    layout (Torch, and the library's own decode with every beam a request of its own) against shared-prefix
    decode at the workload's longest suffix. `ratio` = baseline time / kernel time."""
    import math

    import torch

    import attention_bga_packed_amd as bga
    import comparators as C

    out = {}

    def timed(fn, n=3):
        return timer.span_ms([fn], n) / n

    for name in ("prefill_only", "long_prefill", "long_prefill_1024"):
        if name not in W:
            continue
        w = W[name]
        c, lengths = w["cases"][0], w["lengths"]
        cu = torch.from_numpy(c.cu_seqlens).to(c.q.device)
        sc = 1.0 / math.sqrt(c.d)
        kern = rooflines[name]["avg_launch_us"] / 1e3
        ms = timed(lambda: C.padded_prefill(c.q, c.k, c.v, lengths, sc))
        out[f"{name}/padded_torch"] = {"ms": round(ms, 4), "kernel_ms": round(kern, 4), "ratio": round(ms / kern, 2)}
        if name == "prefill_only":
            ms = timed(lambda: C.packed_prefill(c.q, c.k, c.v, cu, sc))
            out[f"{name}/packed_torch"] = {"ms": round(ms, 4), "kernel_ms": round(kern, 4),
                                           "ratio": round(ms / kern, 2)}
        torch.cuda.empty_cache()
    for name in ("short_decode", "long_beam"):
        if name not in W:
            continue
        w, cfg = W[name], W[name]["cfg"]
        c = w["sets"][0]
        ls = cfg["steps"]
        sc = 1.0 / math.sqrt(cfg["d"])
        kern = rooflines[f"{name}/decode"]["us_per_step"][-1] / 1e3
        R, Wb = cfg["r"], cfg["w"]
        build = timed(lambda: C.per_beam_kv(c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v, ls))
        kt, vf = C.per_beam_kv(c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v, ls)
        ms = timed(lambda: C.per_beam_decode(c.q, kt, vf, sc))
        out[f"{name}/per_beam_torch"] = {"ms": round(ms, 4), "layout_build_ms": round(build, 4),
                                         "kernel_ms": round(kern, 4), "ratio": round(ms / kern, 2),
                                         "suffix_len": ls}
        del kt, vf
        pk, pv = C.per_beam_kv_packed(c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v, ls)
        n = cfg["lp"] + ls
        pcu = torch.arange(0, (R * Wb + 1) * n, n, dtype=torch.int32, device=c.q.device)
        qb = c.q.reshape(R * Wb, 1, *c.q.shape[2:])
        dummy = torch.zeros((R * Wb, 1, 1, cfg["nkv"], cfg["d"]), dtype=torch.bfloat16, device=c.q.device)
        o = torch.empty_like(qb)
        ms = timed(lambda: bga.shared_prefix_decode_packed(qb, pk, pv, pcu, dummy, dummy, 0, out=o, want_lse=False),
                   n=5)
        out[f"{name}/per_beam_own_kernel"] = {"ms": round(ms, 4), "kernel_ms": round(kern, 4),
                                              "ratio": round(ms / kern, 2), "suffix_len": ls}
        del pk, pv
        torch.cuda.empty_cache()
    return out


def workload_config(w):
    cfg = dict(w["cfg"])
    cfg.pop("seed", None)
    if w["kind"] == "loop":
        cfg["generated_tokens"] = w["n_gen"]
        cfg["stop_token"] = 2
    if w["kind"] == "prefill":
        cfg["total_tokens"] = int(sum(w["lengths"]))
        cfg["max_len"] = int(max(w["lengths"]))
        cfg["sequences"] = len(w["lengths"])
        cfg.pop("lengths", None)
    return cfg


def median_of_3(fn):
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(sorted(ts)[1])


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baselines(W, scale):
    """The fp64 oracle (never tuned for speed) on bounded samples of the same inputs, on the host
    cores: median of three runs each, in the units of the GPU figures."""
    import numpy as np

    import oracle
    import workloads as wl

    threads = oracle.num_threads(0)
    model = cpu_model()
    out = {}

    def rec(value, unit, sample, secs):
        return {"value": round(value, 6), "unit": unit, "cores": threads, "kind": "oracle", "sample": sample,
                "seconds_median_of_3": round(secs, 3), "cpu_model": model}

    for name in ("prefill_only", "long_prefill", "long_prefill_1024"):
        if name not in W:
            continue
        w = W[name]
        c, cfg = w["cases"][0], w["cfg"]
        lengths = w["lengths"]
        # bounded sample: the first sequences of the batch up to scale x the 120 x 1024 batch's work (at the
        # default scale every prefill batch is timed whole; about 2 s per run of the 120 x 1024 batch)
        budget = scale * wl.causal_pairs([1024] * 120)
        n, pairs = 0, 0
        while n < len(lengths) and pairs + wl.causal_pairs([lengths[n]]) <= max(budget, wl.causal_pairs(lengths[:1])):
            pairs += wl.causal_pairs([lengths[n]])
            n += 1
        t = int(sum(lengths[:n]))
        q, k, v = c.q[:t].cpu(), c.k[:t].cpu(), c.v[:t].cpu()
        cu = wl.cu_seqlens_from_lengths(lengths[:n])
        secs = median_of_3(lambda: oracle.packed_prefill(q, k, v, cu, nthreads=threads))
        flops = wl.prefill_flops(lengths[:n], cfg["nq"], cfg["d"])
        out[name] = rec(flops / secs / 1e12, "TFLOP/s", f"{n} of {len(lengths)} sequences (T={t}, "
                        f"{cfg['nq']}/{cfg['nkv']} heads, d {cfg['d']}), {flops / 1e9:.1f} GFLOP", secs)
    if "swiglu_fp8" in W:
        cfg = W["swiglu_fp8"]["cfg"]
        x = W["swiglu_fp8"]["fns"][0].__defaults__[0].cpu()
        secs = median_of_3(lambda: oracle.swiglu_quant(x, nthreads=threads))
        b = wl.swiglu_quant_bytes(cfg["tokens"], cfg["inter"])
        out["swiglu_fp8"] = rec(b / secs / 1e9, "GB/s", f"the whole {cfg['tokens']} x {cfg['inter']} input", secs)
    for name in ("short_decode", "long_beam"):
        if name not in W:
            continue
        w, cfg = W[name], W[name]["cfg"]
        c = w["sets"][0]
        ls = cfg["steps"]
        nr = max(1, min(cfg["r"], int(round(scale * cfg["r"]))))
        host = [t[:nr].cpu() for t in (c.q, c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v)]
        secs = median_of_3(lambda: oracle.shared_prefix_decode(*host, ls, nthreads=threads))
        b = wl.decode_bytes(nr, cfg["w"], cfg["nq"], cfg["nkv"], cfg["lp"], ls, cfg["d"])
        out[f"{name}/decode"] = rec(b / secs / 1e9, "GB/s", f"{nr} of {cfg['r']} requests at suffix length {ls}, "
                                    f"{b / 1e6:.1f} MB algorithmic", secs)
        par = w["parents"][ls - 1][:nr].cpu().numpy() if "parents" in w else \
            wl.make_parents(nr, cfg["w"], cfg["w"], seed=1)
        secs = median_of_3(lambda: oracle.suffix_reorder(host[3], host[4], par, ls))
        b = wl.reorder_bytes(nr, cfg["w"], ls, cfg["nkv"], cfg["d"])
        out[f"{name}/reorder"] = rec(b / secs / 1e9, "GB/s", f"{nr} of {cfg['r']} requests at suffix length {ls}",
                                     secs)
        if "topk" in w:
            rows = max(8, min(2 * cfg["w"], int(round(scale * 2 * cfg["w"]))))
            x = w["logits"][0].view(-1, cfg["vocab"])[:rows].unsqueeze(0).cpu()   # the first beam rows of the step
            cum = np.zeros((1, rows), np.float32)
            secs = median_of_3(lambda: oracle.beam_topk(x, cum, 2 * cfg["w"], min(cfg["w"], rows * 2 * cfg["w"]),
                                                        nthreads=threads))
            b = wl.topk_bytes(1, rows, cfg["vocab"], cfg["w"])
            out[f"{name}/topk"] = rec(b / secs / 1e9, "GB/s", f"{rows} of {cfg['r'] * cfg['w']} beam rows over the "
                                      f"full vocabulary, k_local {2 * cfg['w']}", secs)
    return out


if __name__ == "__main__":
    main()
