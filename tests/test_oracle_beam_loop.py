"""Pins for the oracle's fixed-depth beam search (oracle/beam_loop.py), on the CPU.

  * selection: at every step the oracle's candidates, next beams and finished
    hypotheses equal a brute-force beam search that expands every beam by every
    token (all W_in x V candidates ranked at once with numpy's stable lexsort,
    keyed (-score, beam, -logit, token)), then applies the article's 2W rule
    written out again here: stop-token candidates finish, the first W others
    continue;
  * state: every beam's generated K/V rows and token list equal the ones
    rebuilt here by following the recorded parents (lineage bookkeeping
    independent of the oracle's copies), and its attention equals float64 SDPA
    over [prompt; those rows];
  * invariants of the 2W rule: at most one stop-token candidate per source
    beam, W continuing beams that never contain the stop token, finished
    hypotheses that end with it, a final ranking sorted by score.
"""
import importlib.util
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def load_beam_loop():
    """oracle.beam_loop, or the copy named by BGA_ORACLE_BEAM_LOOP (the mutation check plants mistakes there)."""
    path = os.environ.get("BGA_ORACLE_BEAM_LOOP")
    if not path:
        from oracle import beam_loop
        return beam_loop
    spec = importlib.util.spec_from_file_location("oracle._beam_loop_under_test", path)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    return mod


beam_loop = load_beam_loop()


def f32(bits_or_tensor):
    t = bits_or_tensor
    if isinstance(t, torch.Tensor):
        return t.float().numpy()
    return torch.from_numpy(np.ascontiguousarray(t).view(np.int16)).view(torch.bfloat16).float().numpy()


def synthetic_model(R, W, V, nq, nkv, d, eos, seed, eos_boost):
    """Seeded stand-in for the model: per-step query, new K/V and logits; the stop token's logit is raised
    in some rows so that hypotheses finish."""
    cache = {}

    def model(s):
        if s not in cache:
            g = torch.Generator().manual_seed(seed * 100 + s)
            w_in = 1 if s == 0 else W
            x = torch.randn((R, w_in, V), generator=g) * 2.0
            boost = (torch.rand((R, w_in), generator=g) < eos_boost).float() * 6.0
            x[:, :, eos] += boost
            m = {"logits": x.to(torch.bfloat16)}
            if s > 0:
                m["q"] = wl.bf16_normal((R, W, nq, d), g, "cpu")
                m["k"] = wl.bf16_normal((R, W, nkv, d), g, "cpu")
                m["v"] = wl.bf16_normal((R, W, nkv, d), g, "cpu")
            cache[s] = m
        return cache[s]
    return model


def brute_force_step(logits, cum, lse32, W, eos, hist):
    """All W_in x V expansions ranked at once; the 2W best; stop tokens finish, the first W others continue."""
    x = f32(logits)                                   # [W_in, V]
    w_in, V = x.shape
    c = np.zeros(w_in, np.float32) if cum is None else cum
    lp = (x.astype(np.float32) - lse32[:, None].astype(np.float32)).astype(np.float32)
    sc = (c[:, None] + lp).astype(np.float32)
    b = np.repeat(np.arange(w_in), V)
    v = np.tile(np.arange(V), w_in)
    order = np.lexsort((v, -x.ravel(), b, -sc.ravel()))[:2 * W]
    cand = [(int(v[i]), int(b[i]), np.float32(sc.ravel()[i])) for i in order]
    parents, toks, cums, fin = [], [], [], []
    for tok, par, s in cand:
        if tok == eos:
            fin.append((s, hist[par] + [tok]))
        elif len(parents) < W:
            parents.append(par)
            toks.append(hist[par] + [tok])
            cums.append(s)
    return cand, parents, toks, np.array(cums, np.float32), fin


@pytest.mark.parametrize("lengths,W,n_gen,V,eos,boost", [((5, 12, 3), 4, 4, 60, 3, 0.3),
                                                          ((9,), 6, 5, 40, 0, 0.6),
                                                          ((4, 7), 3, 3, 30, 7, 0.0)])
def test_oracle_beam_search_against_brute_force_and_lineage(lengths, W, n_gen, V, eos, boost):
    R, nq, nkv, d = len(lengths), 4, 2, 64
    cu = wl.cu_seqlens_from_lengths(lengths)
    g = torch.Generator().manual_seed(7)
    pk = wl.bf16_normal((int(cu[-1]), nkv, d), g, "cpu")
    pv = wl.bf16_normal((int(cu[-1]), nkv, d), g, "cpu")
    model = synthetic_model(R, W, V, nq, nkv, d, eos, seed=len(lengths) + W, eos_boost=boost)
    records, final = beam_loop.beam_search(pk, pv, cu, model, W, n_gen, eos)
    assert len(records) == n_gen
    scale = 1.0 / np.sqrt(d)
    hist = [[[]] for _ in range(R)]
    cum = None
    lineage = [[[]] for _ in range(R)]         # per beam: the (step, slot) of each generated K/V row
    fin_ref = [[] for _ in range(R)]
    n_finished = 0
    for rec in records:
        s = rec.s
        m = model(s)
        if s > 0:
            for r in range(R):
                for b in range(W):
                    lineage[r][b] = lineage[r][b] + [(s, b)]
                    rows_k = [m2 for m2 in (model(t)["k"][r, slot] for t, slot in lineage[r][b])]
                    rows_v = [m2 for m2 in (model(t)["v"][r, slot] for t, slot in lineage[r][b])]
                    kk = torch.cat([pk[cu[r]:cu[r + 1]]] + [x[None] for x in rows_k]).double()
                    vv = torch.cat([pv[cu[r]:cu[r + 1]]] + [x[None] for x in rows_v]).double()
                    g_ = nq // nkv
                    kk = kk.repeat_interleave(g_, dim=1).transpose(0, 1)
                    vv = vv.repeat_interleave(g_, dim=1).transpose(0, 1)
                    q = m["q"][r, b].double()[:, None, :]
                    ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, scale=scale)[:, 0]
                    assert np.max(np.abs(rec.attn_out[r, b] - ref.numpy())) < 1e-12
        new_hist, new_lin = [], []
        for r in range(R):
            cand, par, toks, c, fin = brute_force_step(m["logits"][r], None if cum is None else cum[r],
                                                       rec.row_lse[r], W, eos, hist[r])
            assert [t for t, _, _ in cand] == list(rec.cand_tokens[r])
            assert [p for _, p, _ in cand] == list(rec.cand_parents[r])
            assert np.array_equal(np.array([x for _, _, x in cand], np.float32), rec.cand_scores[r])
            assert par == list(rec.parents[r]) and toks == rec.tokens[r]
            assert np.array_equal(c, rec.cum[r])
            # invariants of the 2W rule
            stop_parents = [p for t, p, _ in cand if t == eos]
            assert len(stop_parents) == len(set(stop_parents))
            assert all(eos not in t for t in toks)
            fin_ref[r].extend(fin)
            assert [(np.float32(f.score), f.tokens) for f in rec.finished[r]] == fin_ref[r]
            assert all(f.tokens[-1] == eos for f in rec.finished[r])
            new_hist.append(toks)
            new_lin.append([list(lineage[r][p]) for p in par])
        hist, lineage = new_hist, new_lin
        cum = rec.cum
        # the generated K rows of every beam, rebuilt from the lineage
        for r in range(R):
            for b in range(W):
                want = np.stack([wl.bf16_bits(model(t)["k"][r, slot]) for t, slot in lineage[r][b]]) \
                    if lineage[r][b] else np.zeros((0, nkv, d), np.uint16)
                assert np.array_equal(rec.suffix_k[r][b], want)
    for r in range(R):
        n_finished += len(fin_ref[r])
        scores = [sc for sc, _ in final[r]]
        assert scores == sorted(scores, reverse=True)
        assert len(final[r]) == len(fin_ref[r]) + W
    if boost > 0:
        assert n_finished > 0, "the case should exercise finished hypotheses"
