"""The fixed-depth beam search end to end on the GPU (BeamSearch over the
library's calls) against the oracle's beam search, which keeps an explicit
copy of every beam's whole K/V sequence, compared at every step:

  * decode attention output and log-sum-exp (bf16 / LSE tolerances);
  * the 2W global candidates (tokens, parents, scores): bit-exact against the
    oracle run with the GPU's row log-sum-exp (the fp32 value that decides the
    cut); against the oracle's own log-sum-exp only at the cut (<= 4 fp32 ulp);
  * the next beams' parents, token lists and cumulative scores, the finished
    pool, and the reordered suffix K/V (bit for bit against the generated part
    of each beam's explicit K/V);
  * the final ranking of finished hypotheses and beams.

The model between attention and logits is not part of the path: its outputs
(per-step query, the current token's K/V, logits with the stop token raised in
some rows so that hypotheses finish) are drawn from fixed seeds.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import CUT_GAP_ULP, check_bf16, check_lse, cut_gap, say
from oracle import beam_loop

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def synthetic_model(R, W, V, nq, nkv, d, eos, n_gen, seed, boost, std):
    outs = {}
    for s in range(n_gen):
        g = torch.Generator(device=DEV)
        g.manual_seed(seed * 1000 + s)
        w_in = 1 if s == 0 else W
        x = torch.randn((R, w_in, V), generator=g, device=DEV) * std
        x[:, :, eos] += (torch.rand((R, w_in), generator=g, device=DEV) < boost).float() * 3.0 * std
        m = {"logits": x.to(torch.bfloat16)}
        if s > 0:
            m["q"] = wl.bf16_normal((R, W, nq, d), g, DEV)
            m["k"] = wl.bf16_normal((R, W, nkv, d), g, DEV)
            m["v"] = wl.bf16_normal((R, W, nkv, d), g, DEV)
        outs[s] = m
    return outs


def host(t):
    return t.detach().cpu()


@pytest.mark.parametrize("lengths,W,n_gen,V,nq,nkv,d,eos,boost,std", [
    ((5, 40, 130), 8, 5, 1000, 4, 2, 64, 3, 0.3, 2.0),
    ((180, 240, 97, 256), 64, 6, 32000, 16, 8, 128, 151, 0.1, 3.0),
    ((33, 70), 200, 4, 5000, 14, 2, 64, 0, 0.2, 3.0),
    # the long-prompt configuration's beam width and vocabulary: 400 beams of one parent after the first step,
    # scores crowded near the cut (the 8192-entry list and exact cut of the global selection)
    ((64, 200), 400, 4, 151936, 16, 8, 128, 2, 0.05, 3.0),
])
def test_beam_search_steps_against_the_oracle(lengths, W, n_gen, V, nq, nkv, d, eos, boost, std):
    import attention_bga_packed_amd as bga
    from attention_bga_packed_amd.beam_search import BeamSearch

    R = len(lengths)
    cu = wl.cu_seqlens_from_lengths(lengths)
    cu_d = torch.from_numpy(cu).to(DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(R * 31 + W)
    tp = int(cu[-1])
    pq = wl.bf16_normal((tp, nq, d), g, DEV)
    pk = wl.bf16_normal((tp, nkv, d), g, DEV)
    pv = wl.bf16_normal((tp, nkv, d), g, DEV)
    say(f"[beam loop] R={R} prompts {lengths} W={W} N_gen={n_gen} V={V} heads {nq}/{nkv} d {d} stop {eos}")
    # prompt prefill: its K/V is the shared prefix as it is; its last rows would feed the model's head
    p_out, _ = bga.packed_gqa_prefill(pq, pk, pv, cu_d, max(lengths))
    last = bga.last_token_gather(p_out, cu_d)
    assert last.shape == (R, nq, d)
    model = synthetic_model(R, W, V, nq, nkv, d, eos, n_gen, seed=R + W, boost=boost, std=std)

    bs = BeamSearch(R, W, n_gen, V, nq, nkv, d, eos, DEV)
    gpu = []
    cand = bs.start(pk, pv, cu_d, model[0]["logits"])
    torch.cuda.synchronize()
    gpu.append({"cand": {k: host(v) for k, v in cand.items()}, **{k: host(v) if isinstance(v, torch.Tensor) else v
                                                                  for k, v in bs.state.items() if k != "pool"},
                "pool": {k: host(v) for k, v in bs.pool.items()}})
    for s in range(1, n_gen):
        m = model[s]
        out, lse = bs.decode(m["q"], m["k"], m["v"])
        rec = {"attn_out": host(out).clone(), "attn_lse": host(lse).clone()}
        cand = bs.select(m["logits"])
        torch.cuda.synchronize()
        rec["cand"] = {k: host(v) for k, v in cand.items()}
        rec.update({k: host(v) if isinstance(v, torch.Tensor) else v for k, v in bs.state.items() if k != "pool"})
        rec["pool"] = {k: host(v) for k, v in bs.pool.items()}
        gpu.append(rec)
    final = {k: host(v) for k, v in bs.finish().items()}
    torch.cuda.synchronize()

    # the oracle, selecting with the GPU's fp32 row log-sum-exp
    cpu_model = {s: {k: host(v) for k, v in m.items()} for s, m in model.items()}
    records, final_ref = beam_loop.beam_search(host(pk), host(pv), cu, lambda s: cpu_model[s], W, n_gen, eos,
                                               row_lse_for=lambda s: gpu[s]["cand"]["row_lse"].numpy())
    n_fin, worst_gap, n_cut = 0, 0.0, 0
    prev_cum = None
    for s, (g_, o_) in enumerate(zip(gpu, records)):
        if s > 0:
            check_bf16(g_["attn_out"], o_.attn_out, f"step {s} attention")
            check_lse(g_["attn_lse"], o_.attn_lse, f"step {s} attention")
        for key, ref in (("tokens", o_.cand_tokens), ("parents", o_.cand_parents), ("scores", o_.cand_scores)):
            assert np.array_equal(g_["cand"][key].numpy(), ref), f"step {s}: candidate {key}"
        # the oracle's own log-sum-exp: the selection may differ only at the cut
        logits = cpu_model[s]["logits"]
        own = oracle.beam_topk(logits, prev_cum, 2 * W, 2 * W)
        given = oracle.beam_topk(logits, prev_cum, 2 * W, 2 * W, row_lse=g_["cand"]["row_lse"].numpy())
        assert np.abs(g_["cand"]["row_lse"].numpy().astype(np.float64) - own["row_lse64"]).max() <= 1e-5
        for r in range(R):
            if not (np.array_equal(own["tokens"][r], given["tokens"][r]) and
                    np.array_equal(own["parents"][r], given["parents"][r])):
                gap, drift = cut_gap(given, own, r, 2 * W, 2 * W)
                assert gap <= CUT_GAP_ULP and drift <= CUT_GAP_ULP, (s, r, gap, drift)
                worst_gap, n_cut = max(worst_gap, gap), n_cut + 1
        prev_cum = o_.cum
        # the next beams
        assert np.array_equal(g_["parents"].numpy(), o_.parents), f"step {s}: parents"
        assert np.array_equal(g_["cum"].numpy(), o_.cum), f"step {s}: cumulative scores"
        toks = g_["tokens"].numpy()
        for r in range(R):
            for b in range(W):
                assert list(toks[r, b, :s + 1]) == o_.tokens[r][b], (s, r, b)
                if s > 0:
                    assert np.array_equal(wl.bf16_bits(g_["suffix_k"][r, b, :s]), o_.suffix_k[r][b]), (s, r, b)
                    assert np.array_equal(wl.bf16_bits(g_["suffix_v"][r, b, :s]), o_.suffix_v[r][b]), (s, r, b)
            fin = o_.finished[r]
            pool = g_["pool"]
            assert int(pool["count"][r]) == len(fin), (s, r)
            for i, f in enumerate(fin):
                assert np.float32(pool["scores"][r, i]) == np.float32(f.score)
                assert int(pool["lengths"][r, i]) == len(f.tokens)
                assert list(pool["tokens"][r, i, :len(f.tokens)].numpy()) == f.tokens
    for r in range(R):
        n = int(final["count"][r])
        assert n == len(final_ref[r])
        n_fin += n - W
        for i, (sc, toks) in enumerate(final_ref[r]):
            assert np.float32(final["scores"][r, i]) == sc, (r, i)
            ln = int(final["lengths"][r, i])
            assert list(final["tokens"][r, i, :ln].numpy()) == toks, (r, i)
    say(f"    {n_gen} steps identical; finished hypotheses {n_fin}; requests whose own-lse selection differs at "
        f"the cut: {n_cut} (largest gap {worst_gap:.2f} ulp)")
    assert boost == 0 or n_fin > 0


def test_beam_search_replays_as_a_graph():
    """The whole loop allocates nothing, clears nothing and never waits on the host once its state exists, so it
    can be captured once (HIP stream capture through torch.cuda.graph) and replayed: every replay, with eager work
    and synchronisations between them, gives the final ranking of the eager loop bit for bit."""
    from attention_bga_packed_amd.beam_search import BeamSearch

    lengths, W, n_gen, V, nq, nkv, d, eos = (40, 130), 16, 5, 3000, 8, 4, 64, 3
    R = len(lengths)
    cu = torch.from_numpy(wl.cu_seqlens_from_lengths(lengths)).to(DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    tp = sum(lengths)
    pk = wl.bf16_normal((tp, nkv, d), g, DEV)
    pv = wl.bf16_normal((tp, nkv, d), g, DEV)
    model = synthetic_model(R, W, V, nq, nkv, d, eos, n_gen, seed=17, boost=0.2, std=3.0)
    bs = BeamSearch(R, W, n_gen, V, nq, nkv, d, eos, DEV)

    def loop():
        bs.start(pk, pv, cu, model[0]["logits"])
        for s in range(1, n_gen):
            m = model[s]
            bs.decode(m["q"], m["k"], m["v"])
            bs.select(m["logits"])
        return bs.finish()

    say(f"[beam loop graph] R={R} W={W} N_gen={n_gen} V={V}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # eager runs (the first one sizes the final ranking's buffers)
        loop()
        ref = {k: v.clone() for k, v in loop().items()}
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in bs.final.values():
            t.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: host(v) for k, v in bs.final.items()}
        want = {k: host(v) for k, v in ref.items()}
        assert torch.equal(got["count"], want["count"]), rep
        for r in range(R):   # the ranking fills the first count entries of each request
            n = int(want["count"][r])
            assert torch.equal(got["scores"][r, :n], want["scores"][r, :n]), (rep, r)
            assert torch.equal(got["lengths"][r, :n], want["lengths"][r, :n]), (rep, r)
            for i in range(n):
                ln = int(want["lengths"][r, i])
                assert torch.equal(got["tokens"][r, i, :ln], want["tokens"][r, i, :ln]), (rep, r, i)
        assert torch.randn(256, device=DEV).abs().sum().item() > 0   # eager work between replays
