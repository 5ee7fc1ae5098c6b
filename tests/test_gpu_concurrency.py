"""The library keeps no state between calls and may be called from several
host threads at once, each on its own stream (the ownership rules of the C
ABI): two threads issue prefill, decode, top-K and reorder calls on two
streams concurrently, and every result must be bit-identical to the same call
made alone on the default stream."""
import threading

import pytest
import torch

import workloads as wl
from helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_two_threads_two_streams_match_calls_made_alone():
    import attention_bga_packed_amd as bga

    pc = wl.make_prefill_case([300, 64, 513, 7], 14, 2, 64, seed=71, device=DEV)
    cu = torch.from_numpy(pc.cu_seqlens).to(DEV)
    dc = wl.make_decode_case(2, 64, 200, 4, 16, 8, 128, seed=72, device=DEV)
    logits = wl.make_logits(2, 64, 32000, 3.0, seed=73, device=DEV)
    cum = (torch.arange(128, device=DEV, dtype=torch.float32).reshape(2, 64) * -0.01).contiguous()
    parent = torch.from_numpy(wl.make_parents(2, 64, 64, seed=74)).to(DEV)

    calls = {
        "prefill": lambda: bga.packed_gqa_prefill(pc.q, pc.k, pc.v, cu, 513),
        "decode": lambda: bga.shared_prefix_decode(dc.q, dc.prefix_k, dc.prefix_v, dc.suffix_k, dc.suffix_v, 3),
        "topk": lambda: tuple(bga.beam_topk(logits, cum, 128, 64).values()),
        "reorder": lambda: bga.suffix_reorder(dc.suffix_k, dc.suffix_v, parent, 3),
    }
    torch.cuda.synchronize()
    ref = {name: tuple(t.clone() for t in fn()) for name, fn in calls.items()}
    torch.cuda.synchronize()

    plans = [["prefill", "topk", "decode", "reorder"] * 6, ["decode", "reorder", "prefill", "topk"] * 6]
    results = [[], []]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()   # default priority
            with torch.cuda.stream(s):
                for name in plans[i]:
                    results[i].append((name, tuple(t.clone() for t in calls[name]())))
            s.synchronize()
        except Exception as e:   # surfaced in the main thread
            errors.append(e)

    say("[concurrency] two host threads, two streams, 24 calls each")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        assert len(results[i]) == len(plans[i])
        for name, outs in results[i]:
            for got, want in zip(outs, ref[name]):
                assert torch.equal(got, want), (i, name)
