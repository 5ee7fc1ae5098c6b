"""Pins for the fp64 oracle: it is checked against facts other than itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, a wrong head or position index, a transposed operand, a wrong tie
rule) fails at least one of them:

  * brute-force padded attention with an explicit [B, L_max, L_max] mask (numpy);
  * the library routine torch.nn.functional.scaled_dot_product_attention in
    float64, with K/V heads expanded (a different formulation of GQA);
  * scipy.special.logsumexp for every log-sum-exp;
  * closed forms (first token of a sequence, constant value rows);
  * the article's invariants (packed == per-sequence, sequence isolation,
    shared-prefix == attention over the explicit concatenation, pruning lemma,
    monotonicity of log-softmax);
  * numpy's stable lexsort for every ranking with its tie rule.
"""
import json
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f64(bits):
    """bf16 bits -> float64, via torch's own bfloat16 decoding (not the oracle's)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def tiny_case(lengths=(5, 17, 40), nq=4, nkv=2, d=64, seed=0):
    return wl.make_prefill_case(list(lengths), nq, nkv, d, seed)


# ---------------------------------------------------------------- C-1 prefill

def brute_force_padded(case, scale):
    """Pad every sequence to L_max; mask = same sequence and key <= query."""
    q, k, v = (f64(wl.bf16_bits(x)) for x in (case.q, case.k, case.v))
    lens = case.lengths
    b, lmax = len(lens), max(lens)
    nq, nkv, d = case.nq, case.nkv, case.d
    g = nq // nkv
    qp = np.zeros((b, lmax, nq, d)); kp = np.zeros((b, lmax, nkv, d)); vp = np.zeros((b, lmax, nkv, d))
    valid = np.zeros((b, lmax), bool)
    for i, (s, n) in enumerate(zip(case.cu_seqlens[:-1], lens)):
        qp[i, :n], kp[i, :n], vp[i, :n] = q[s:s + n], k[s:s + n], v[s:s + n]
        valid[i, :n] = True
    pos = np.arange(lmax)
    mask = (pos[None, :, None] >= pos[None, None, :]) & valid[:, None, :] & valid[:, :, None]  # [b, t, u]
    out = np.zeros_like(qp); lse = np.zeros((b, lmax, nq))
    for h in range(nq):
        kh, vh = kp[:, :, h // g], vp[:, :, h // g]
        s = scale * np.einsum("btd,bud->btu", qp[:, :, h], kh)
        s = np.where(mask, s, -np.inf)
        s[~valid] = 0.0  # padded query rows: anything finite, dropped below
        m = s.max(-1, keepdims=True)
        p = np.exp(s - m)
        out[:, :, h] = np.einsum("btu,bud->btd", p, vh) / p.sum(-1, keepdims=True)
        lse[:, :, h] = (m[..., 0] + np.log(p.sum(-1)))
    o_packed = np.concatenate([out[i, :n] for i, n in enumerate(lens)])
    l_packed = np.concatenate([lse[i, :n] for i, n in enumerate(lens)])
    return o_packed, l_packed


def test_prefill_matches_padded_brute_force():
    case = tiny_case()
    scale = 1.0 / np.sqrt(case.d)
    o, lse = oracle.packed_prefill(case.q, case.k, case.v, case.cu_seqlens, scale)
    ob, lb = brute_force_padded(case, scale)
    assert np.max(np.abs(o - ob)) < 1e-12
    assert np.max(np.abs(lse - lb)) < 1e-12


@pytest.mark.parametrize("nq,nkv", [(4, 2), (14, 2), (3, 3), (8, 1)])
def test_prefill_matches_library_sdpa(nq, nkv):
    """torch SDPA (float64, causal, K/V repeated per group) per sequence."""
    case = tiny_case(lengths=(1, 9, 33), nq=nq, nkv=nkv, d=64, seed=11)
    scale = 1.0 / np.sqrt(case.d)
    o, lse = oracle.packed_prefill(case.q, case.k, case.v, case.cu_seqlens, scale)
    g = nq // nkv
    for s, n in zip(case.cu_seqlens[:-1], case.lengths):
        q = case.q[s:s + n].double().transpose(0, 1)                      # [nq, n, d]
        k = case.k[s:s + n].double().repeat_interleave(g, dim=1).transpose(0, 1)
        v = case.v[s:s + n].double().repeat_interleave(g, dim=1).transpose(0, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
        assert np.max(np.abs(o[s:s + n] - ref.transpose(0, 1).numpy())) < 1e-12
        scores = scale * (q @ k.transpose(1, 2)).numpy()
        scores = np.where(np.tril(np.ones((n, n), bool)), scores, -np.inf)
        assert np.max(np.abs(lse[s:s + n] - logsumexp(scores, axis=-1).T)) < 1e-12


def test_prefill_first_token_closed_form():
    case = tiny_case()
    scale = 0.37
    o, lse = oracle.packed_prefill(case.q, case.k, case.v, case.cu_seqlens, scale)
    q, k, v = (f64(wl.bf16_bits(x)) for x in (case.q, case.k, case.v))
    g = case.nq // case.nkv
    for s in case.cu_seqlens[:-1]:
        for h in range(case.nq):
            assert np.array_equal(o[s, h], v[s, h // g])
            assert abs(lse[s, h] - scale * np.dot(q[s, h], k[s, h // g])) < 1e-12


def test_prefill_constant_values_give_that_row():
    case = tiny_case()
    row = torch.randn(case.d).to(torch.bfloat16)
    case.v[:] = row
    o, _ = oracle.packed_prefill(case.q, case.k, case.v, case.cu_seqlens)
    assert np.max(np.abs(o - row.double().numpy())) < 1e-12


def test_packed_equals_separate_sequences():
    case = tiny_case()
    o, lse = oracle.packed_prefill(case.q, case.k, case.v, case.cu_seqlens)
    for s, n in zip(case.cu_seqlens[:-1], case.lengths):
        cu = np.array([0, n], np.int32)
        oi, li = oracle.packed_prefill(case.q[s:s + n], case.k[s:s + n], case.v[s:s + n], cu)
        assert np.array_equal(oi, o[s:s + n]) and np.array_equal(li, lse[s:s + n])


def test_sequence_isolation():
    case = tiny_case()
    o, lse = oracle.packed_prefill(case.q, case.k, case.v, case.cu_seqlens)
    s, n = case.cu_seqlens[1], case.lengths[1]
    for t in (case.q, case.k, case.v):
        t[s:s + n] = -t[s:s + n] + 0.5
    o2, l2 = oracle.packed_prefill(case.q, case.k, case.v, case.cu_seqlens)
    keep = np.ones(len(o), bool); keep[s:s + n] = False
    assert np.array_equal(o[keep], o2[keep]) and np.array_equal(lse[keep], l2[keep])
    assert not np.array_equal(o[~keep], o2[~keep])


def test_zero_length_sequences_produce_no_rows():
    case = tiny_case(lengths=(0, 7, 0, 3, 0))
    o, lse = oracle.packed_prefill(case.q, case.k, case.v, case.cu_seqlens)
    o2, l2 = oracle.packed_prefill(case.q, case.k, case.v, np.array([0, 7, 10], np.int32))
    assert o.shape[0] == 10 and np.array_equal(o, o2) and np.array_equal(lse, l2)


# ---------------------------------------------------------- C-2 shared prefix

def small_decode(r=2, w=5, lp=7, ls_cap=3, nq=4, nkv=2, d=64, seed=21):
    return wl.make_decode_case(r, w, lp, ls_cap, nq, nkv, d, seed)


@pytest.mark.parametrize("ls,w", [(0, 5), (1, 5), (3, 5), (2, 1)])
def test_decode_matches_sdpa_over_concat(ls, w):
    """SDPA (float64) over the explicit [prompt; suffix] of every beam; W = 1 is
    ordinary single-sequence decode."""
    c = small_decode(w=w)
    scale = 1.0 / np.sqrt(c.d)
    o, lse = oracle.shared_prefix_decode(c.q, c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v, ls, scale)
    g = c.nq // c.nkv
    for r in range(c.r):
        for b in range(c.w):
            kc = torch.cat([c.prefix_k[r], c.suffix_k[r, b, :ls]]).double()   # [n, nkv, d]
            vc = torch.cat([c.prefix_v[r], c.suffix_v[r, b, :ls]]).double()
            kc = kc.repeat_interleave(g, dim=1).transpose(0, 1)                # [nq, n, d]
            vc = vc.repeat_interleave(g, dim=1).transpose(0, 1)
            q = c.q[r, b].double()[:, None, :]                                 # [nq, 1, d]
            ref = torch.nn.functional.scaled_dot_product_attention(q, kc, vc, scale=scale)[:, 0]
            assert np.max(np.abs(o[r, b] - ref.numpy())) < 1e-12
            sc = scale * (q @ kc.transpose(1, 2))[:, 0].numpy()
            assert np.max(np.abs(lse[r, b] - logsumexp(sc, axis=-1))) < 1e-12


def test_decode_equals_last_row_of_causal_prefill():
    """Decode over [prefix; suffix_b] equals the last query row of causal prefill
    over the sequence prefix + suffix_b with q_b placed at the last position."""
    c = small_decode(r=1, w=3, lp=6, ls_cap=2)
    ls = 2
    o, lse = oracle.shared_prefix_decode(c.q, c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v, ls)
    for b in range(c.w):
        n = c.lp + ls
        k = torch.cat([c.prefix_k[0], c.suffix_k[0, b, :ls]])
        v = torch.cat([c.prefix_v[0], c.suffix_v[0, b, :ls]])
        q = torch.zeros((n, c.nq, c.d), dtype=torch.bfloat16)
        q[-1] = c.q[0, b]
        op, lp_ = oracle.packed_prefill(q, k, v, np.array([0, n], np.int32))
        assert np.max(np.abs(op[-1] - o[0, b])) < 1e-12
        assert np.max(np.abs(lp_[-1] - lse[0, b])) < 1e-12


def test_decode_beam_permutation_equivariance():
    c = small_decode()
    o, lse = oracle.shared_prefix_decode(c.q, c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v, 2)
    perm = torch.tensor([3, 0, 4, 1, 2])
    o2, l2 = oracle.shared_prefix_decode(c.q[:, perm], c.prefix_k, c.prefix_v, c.suffix_k[:, perm],
                                         c.suffix_v[:, perm], 2)
    assert np.array_equal(o2, o[:, perm.numpy()]) and np.array_equal(l2, lse[:, perm.numpy()])


def packed_prompt_case(lps=(7, 0, 3), w=5, ls_cap=3, nq=4, nkv=2, d=64, seed=23):
    """Prompts of different lengths packed back to back [sum Lp, Nkv, D], plus per-beam suffixes."""
    c = wl.make_decode_case(len(lps), w, 1, ls_cap, nq, nkv, d, seed)
    gen = torch.Generator().manual_seed(seed + 1)
    tp = int(sum(lps))
    pk = wl.bf16_normal((tp, nkv, d), gen, "cpu")
    pv = wl.bf16_normal((tp, nkv, d), gen, "cpu")
    return c, pk, pv, wl.cu_seqlens_from_lengths(lps)


@pytest.mark.parametrize("lps,ls,w", [((7, 0, 3), 2, 5), ((1, 9), 0, 3), ((4, 4, 4), 1, 1), ((0, 2), 3, 2)])
def test_decode_packed_prompts_match_sdpa_over_concat(lps, ls, w):
    """Prompts of their own lengths (0 included when the suffix is not empty), kept packed: SDPA (float64)
    over the explicit [prompt of r; suffix of beam b] of every beam; W = 1 is ordinary decode."""
    c, pk, pv, cu = packed_prompt_case(lps, w)
    scale = 1.0 / np.sqrt(c.d)
    o, lse = oracle.shared_prefix_decode_packed(c.q, pk, pv, cu, c.suffix_k, c.suffix_v, ls, scale)
    g = c.nq // c.nkv
    for r in range(c.r):
        for b in range(c.w):
            kc = torch.cat([pk[cu[r]:cu[r + 1]], c.suffix_k[r, b, :ls]]).double()
            vc = torch.cat([pv[cu[r]:cu[r + 1]], c.suffix_v[r, b, :ls]]).double()
            kc = kc.repeat_interleave(g, dim=1).transpose(0, 1)
            vc = vc.repeat_interleave(g, dim=1).transpose(0, 1)
            q = c.q[r, b].double()[:, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(q, kc, vc, scale=scale)[:, 0]
            assert np.max(np.abs(o[r, b] - ref.numpy())) < 1e-12
            sc = scale * (q @ kc.transpose(1, 2))[:, 0].numpy()
            assert np.max(np.abs(lse[r, b] - logsumexp(sc, axis=-1))) < 1e-12


def test_decode_packed_prompt_rejects_a_beam_without_keys():
    c, pk, pv, cu = packed_prompt_case((3, 0), 2)
    with pytest.raises(ValueError):
        oracle.shared_prefix_decode_packed(c.q, pk, pv, cu, c.suffix_k, c.suffix_v, 0)


def test_last_token_gather_matches_fancy_indexing():
    lengths = [3, 0, 1, 7, 0, 2]
    cu = wl.cu_seqlens_from_lengths(lengths)
    x = np.random.default_rng(4).integers(0, 1 << 16, (int(cu[-1]), 5, 6)).astype(np.uint16)
    y = oracle.last_token_gather(x, cu)
    for i, n in enumerate(lengths):
        if n:
            assert np.array_equal(y[i], x[cu[i + 1] - 1])
        else:
            assert not y[i].any()
    # every sequence of one token: the gather is the identity
    ones = wl.cu_seqlens_from_lengths([1] * 6)
    z = np.arange(6 * 8, dtype=np.float32).reshape(6, 8)
    assert np.array_equal(oracle.last_token_gather(z, ones), z)


# ------------------------------------------------------------- C-3 reorder

def test_reorder_identity_and_gather():
    c = small_decode()
    ident = np.tile(np.arange(c.w, dtype=np.int32), (c.r, 1))
    dk, dv = oracle.suffix_reorder(c.suffix_k, c.suffix_v, ident, c.ls_cap)
    assert np.array_equal(dk, wl.bf16_bits(c.suffix_k)) and np.array_equal(dv, wl.bf16_bits(c.suffix_v))
    par = wl.make_parents(c.r, c.w, c.w, seed=3)
    tok = np.random.default_rng(0).integers(0, 1000, (c.r, c.w, 6)).astype(np.int32)
    dk, dv, dt = oracle.suffix_reorder(c.suffix_k, c.suffix_v, par, 2, tok, 4)
    sk, sv = wl.bf16_bits(c.suffix_k), wl.bf16_bits(c.suffix_v)
    ridx = np.arange(c.r)[:, None]
    assert np.array_equal(dk[:, :, :2], sk[ridx, par][:, :, :2])
    assert np.array_equal(dv[:, :, :2], sv[ridx, par][:, :, :2])
    assert not dk[:, :, 2:].any()
    assert np.array_equal(dt[:, :, :4], tok[ridx, par][:, :, :4]) and not dt[:, :, 4:].any()


def test_multistep_reorder_equals_per_beam_full_kv():
    """Shared prefix + reordered suffix gives the same attention as every beam
    holding its own full K/V copy (the W*(L_p+L_s) layout) through 3 steps."""
    r, w, lp, steps, nq, nkv, d = 1, 4, 5, 3, 2, 1, 64
    c = wl.make_decode_case(r, w, lp, steps, nq, nkv, d, seed=5)
    gen = torch.Generator().manual_seed(9)
    sk = torch.zeros_like(c.suffix_k); sv = torch.zeros_like(c.suffix_v)
    full_k = [[c.prefix_k[0].clone()] for _ in range(w)]
    full_v = [[c.prefix_v[0].clone()] for _ in range(w)]
    for step in range(1, steps + 1):
        newk = wl.bf16_normal((r, w, nkv, d), gen, "cpu"); newv = wl.bf16_normal((r, w, nkv, d), gen, "cpu")
        sk[:, :, step - 1] = newk; sv[:, :, step - 1] = newv
        for b in range(w):
            full_k[b].append(newk[0, b][None]); full_v[b].append(newv[0, b][None])
        q = wl.bf16_normal((r, w, nq, d), gen, "cpu")
        o, _ = oracle.shared_prefix_decode(q, c.prefix_k, c.prefix_v, sk, sv, step)
        for b in range(w):
            kk = torch.cat(full_k[b]); vv = torch.cat(full_v[b])
            of, _ = oracle.packed_prefill(torch.cat([torch.zeros((kk.shape[0] - 1, nq, d), dtype=torch.bfloat16),
                                                     q[0, b][None]]), kk, vv, np.array([0, kk.shape[0]], np.int32))
            assert np.max(np.abs(of[-1] - o[0, b])) < 1e-12
        par = wl.make_parents(r, w, w, seed=100 + step)
        dk, dv = oracle.suffix_reorder(sk, sv, par, step)
        sk = torch.from_numpy(dk.view(np.int16)).view(torch.bfloat16)
        sv = torch.from_numpy(dv.view(np.int16)).view(torch.bfloat16)
        full_k = [[t.clone() for t in full_k[p]] for p in par[0]]
        full_v = [[t.clone() for t in full_v[p]] for p in par[0]]


# --------------------------------------------------------------- C-4 top-K

def topk_inputs(r=2, w=3, vocab=300, std=3.0, seed=7, cum=True):
    x = wl.make_logits(r, w, vocab, std, seed)
    c = (np.random.default_rng(seed).standard_normal((r, w)) * 4 - 10).astype(np.float32) if cum else None
    return x, c


def brute_force_single_stage(x_bits, cum, k_global):
    """Score every (beam, token) pair, rank all of them at once by
    (-score, beam, -logit, token), keep k_global."""
    x = f64(x_bits).astype(np.float32)
    r, w, vocab = x.shape
    lse32 = np.float32(logsumexp(x.astype(np.float64), axis=-1)).astype(np.float32)
    c = np.zeros((r, w), np.float32) if cum is None else cum
    out = []
    for i in range(r):
        lp = x[i] - lse32[i][:, None]                 # float32 arithmetic
        s = c[i][:, None] + lp                        # float32 arithmetic
        beam = np.repeat(np.arange(w), vocab); tok = np.tile(np.arange(vocab), w)
        order = np.lexsort((tok, -x[i].ravel(), beam, -s.ravel()))[:k_global]
        out.append((tok[order], beam[order], s.ravel()[order]))
    return out


@pytest.mark.parametrize("k_local,k_global", [(6, 3), (6, 6), (10, 4), (1, 1)])
def test_topk_pruning_lemma_and_scores(k_local, k_global):
    x, cum = topk_inputs()
    res = oracle.beam_topk(x, cum, k_local, k_global)
    bf = brute_force_single_stage(wl.bf16_bits(x), cum, k_global)
    for i, (tok, beam, s) in enumerate(bf):
        assert np.array_equal(res["tokens"][i], tok)
        assert np.array_equal(res["parents"][i], beam)
        assert np.array_equal(res["scores"][i], s)


def test_topk_ties_straddle_the_cut():
    """Coarse logits force many equal values; lower ids must win every tie."""
    gen = torch.Generator().manual_seed(1)
    x = torch.randint(-3, 4, (2, 4, 200), generator=gen).to(torch.bfloat16)
    cum = np.array([[0, 0, -1, 0], [-2, -2, -2, -2]], np.float32)
    for k_local, k_global in [(8, 4), (8, 8), (30, 16)]:
        res = oracle.beam_topk(x, cum, k_local, k_global)
        bf = brute_force_single_stage(wl.bf16_bits(x), cum, k_global)
        for i, (tok, beam, s) in enumerate(bf):
            assert np.array_equal(res["tokens"][i], tok) and np.array_equal(res["parents"][i], beam)


def test_topk_stage1_is_stable_sort_and_lse():
    x, cum = topk_inputs(vocab=500)
    k_local = 17
    res = oracle.beam_topk(x, cum, k_local, 5)
    xf = f64(wl.bf16_bits(x))
    for i in range(x.shape[0]):
        for b in range(x.shape[1]):
            order = np.lexsort((np.arange(xf.shape[-1]), -xf[i, b]))[:k_local]
            assert np.array_equal(res["local_tokens"][i, b], order)
            lse64 = logsumexp(xf[i, b])
            assert abs(res["row_lse64"][i, b] - lse64) < 1e-12
            assert res["row_lse"][i, b] == np.float32(lse64)
            # monotonicity: the same ids rank first by fp64 log-probability
            lp = xf[i, b] - lse64
            assert np.array_equal(np.lexsort((np.arange(lp.size), -lp))[:k_local], order)


def test_topk_full_vocab_probabilities_sum_to_one():
    x, _ = topk_inputs(r=1, w=2, vocab=64)
    res = oracle.beam_topk(x, None, 64, 2)
    lp = res["local_scores"].astype(np.float64)
    assert np.all(np.abs(np.exp(lp).sum(-1) - 1.0) < 1e-6)
    xf = f64(wl.bf16_bits(x))
    for b in range(2):
        assert np.array_equal(res["local_tokens"][0, b], np.lexsort((np.arange(64), -xf[0, b])))


def test_topk_all_equal_logits():
    x = torch.full((1, 3, 50), 1.5, dtype=torch.bfloat16)
    res = oracle.beam_topk(x, np.zeros((1, 3), np.float32), 8, 5)
    assert np.array_equal(res["local_tokens"][0], np.tile(np.arange(8), (3, 1)))
    assert np.array_equal(res["parents"][0], np.zeros(5)) and np.array_equal(res["tokens"][0], np.arange(5))


def test_topk_negative_zero_equals_positive_zero():
    x = torch.tensor([[[0.0, -0.0, 0.0, -1.0, -0.0]]], dtype=torch.bfloat16)
    x[0, 0, 1] = -0.0
    res = oracle.beam_topk(x, None, 4, 2)
    assert list(res["local_tokens"][0, 0]) == [0, 1, 2, 4]


# -------------------------------------------------------------- work counts

def test_triangular_counts_match_printed_example():
    g = json.load(open(os.path.join(GOLDEN, "triangular_qk_counts.json")))
    for case in g["cases"]:
        assert wl.causal_pairs(case["lengths"]) == case["qk_dots"]
    for case in g["approximate"]:
        assert abs(wl.causal_pairs(case["lengths"]) / case["qk_dots_about"] - 1) < 0.01
    # logical FLOPs: 2 matmuls x 2 FLOPs per MAC x D per pair and head
    assert wl.prefill_flops([5, 17, 40], 4, 64) == 4 * 64 * 4 * 988


def test_effective_mfu_matches_printed_shares():
    g = json.load(open(os.path.join(GOLDEN, "effective_mfu.json")))
    pk = g["peaks_tflops"]
    for row in g["rows"]:
        f = row["tflop_per_request"]
        bf = wl.effective_mfu(row["qps"], f["bf16"], pk["bf16"])
        f8 = wl.effective_mfu(row["qps"], 0.0, 1.0, f["fp8"], pk["fp8"])
        assert abs(100 * bf - row["share_pct"]["bf16"]) <= 1.5
        assert abs(100 * f8 - row["share_pct"]["fp8"]) <= 1.5
        assert abs(100 * (bf + f8) - row["total_pct"]) <= 3.0  # two rounded shares


def test_state_size_shared_prefix_vs_per_beam():
    # one prompt copy plus W short suffixes vs W full copies
    assert wl.state_elems_shared_prefix(480, 400, 5, 8, 128) == (480 + 400 * 5) * 8 * 128
    assert wl.state_elems_per_beam(480, 400, 5, 8, 128) == 400 * (480 + 5) * 8 * 128
    assert wl.decode_bytes(32, 100, 16, 8, 128, 1, 64) == 28_254_208


def test_beam_topk_given_lse_reproduces_own_lse():
    """Supplying the oracle's own fp32 row log-sum-exp reproduces its outputs
    bit for bit; a shifted log-sum-exp shifts every stage-1 score by one fp32
    subtraction and leaves the stage-1 ids unchanged."""
    x = wl.make_logits(2, 4, 700, 2.0, seed=31)
    cum = np.array([[0, -1, -2, -3], [-0.5, -0.25, 0, -4]], np.float32)
    a = oracle.beam_topk(x, cum, 12, 6)
    b = oracle.beam_topk(x, cum, 12, 6, row_lse=a["row_lse"])
    for key in ("local_tokens", "local_scores", "tokens", "parents", "scores"):
        assert np.array_equal(a[key], b[key]), key
    shifted = (a["row_lse"] + np.float32(0.5)).astype(np.float32)
    c = oracle.beam_topk(x, cum, 12, 6, row_lse=shifted)
    assert np.array_equal(c["local_tokens"], a["local_tokens"])
    xs = x.float().numpy()
    lp = np.take_along_axis(xs, c["local_tokens"], axis=2) - shifted[:, :, None]
    assert np.array_equal(c["local_scores"], cum[:, :, None] + lp)
