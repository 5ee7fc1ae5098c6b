"""Fixed-depth beam search, written out plainly — TEST INFRASTRUCTURE ONLY (oracle).

The article's bounded generation (section 2.3, the loop of "prompt prefill ->
first-step candidate initialisation -> (N_gen - 1) x [decode -> per-beam
candidate selection -> cumulative score merge -> parent index update -> token
and suffix K/V reorder] -> final candidates and scores") and its candidate rule
(section 3.3: 2W global candidates are kept so that hypotheses that produced the
stop token can finish while W beams continue).

This oracle keeps the simplest state there is: every beam owns an explicit
copy of its whole K/V sequence (prompt + generated tokens, the W (L_p + L_s)
layout the article's shared-prefix layout replaces) and its own token list.
The arithmetic of each step is the oracle's C functions: attention of one query
over an explicit K/V list (oracle.shared_prefix_decode_packed with every beam
its own "request" of one beam and no suffix) and the two-stage selection
(oracle.beam_topk with k_local = k_global = 2W). The stop-token split and the
final ranking are plain Python loops.

Readings (where the pages leave the step open):
  * the model between attention and logits is not part of the path: its
    outputs (per-step query, the new token's K/V, the logits) are inputs here,
    drawn synthetically by the caller;
  * step 0 selects from the prompt's last-token logits [R, 1, V] with zero
    cumulative score; decode step s (1 .. N_gen-1) first gives each beam the K/V
    of its current (last selected) token, so the suffix holds s tokens;
  * of the 2W global candidates (best first), every stop-token candidate
    becomes a finished hypothesis (its tokens end with the stop token) and the
    first W others become the next beams, in candidate order; each source beam
    has at most one stop-token candidate, so at least W others always remain;
  * after the last step the finished hypotheses and the W beams are ranked
    together by cumulative score (no length normalisation: the pages name
    none), ties to the earlier-finished, then to the lower beam.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import beam_topk, shared_prefix_decode_packed, _bits


@dataclass
class Finished:
    score: float
    tokens: list


@dataclass
class StepRecord:
    """What one step produced (s = 0 is the first-step initialisation)."""
    s: int
    attn_out: np.ndarray | None        # [R, W, Nq, D] fp64 (decode steps)
    attn_lse: np.ndarray | None        # [R, W, Nq]
    cand_tokens: np.ndarray            # [R, 2W] the global candidates, best first
    cand_parents: np.ndarray
    cand_scores: np.ndarray
    row_lse: np.ndarray                # [R, W_in] fp32
    parents: np.ndarray                # [R, W] source beam of each next beam
    tokens: list                       # [R][W] token lists of the next beams
    cum: np.ndarray                    # [R, W] fp32 cumulative scores of the next beams
    suffix_k: list                     # [R][W] generated-token K rows [s, Nkv, D] (uint16 bits)
    suffix_v: list
    finished: list = field(default_factory=list)   # [R] list of Finished so far


def advance(cand_tokens, cand_parents, cand_scores, W, eos, histories):
    """The article's 2W rule for one request: stop-token candidates finish, the first W others continue.
    histories[b] is source beam b's token list. Returns (parents, tokens, cum, finished)."""
    parents, tokens, cum, finished = [], [], [], []
    for tok, par, sc in zip(cand_tokens, cand_parents, cand_scores):
        tok, par = int(tok), int(par)
        if tok == eos:
            finished.append(Finished(float(sc), list(histories[par]) + [tok]))
        elif len(parents) < W:
            parents.append(par)
            tokens.append(list(histories[par]) + [tok])
            cum.append(np.float32(sc))
    assert len(parents) == W, "fewer than W continuing candidates"
    return parents, tokens, np.array(cum, np.float32), finished


def final_ranking(finished, cum, tokens):
    """Finished hypotheses and the last beams, best first (score desc; ties: finished before beams, earlier
    finished first, lower beam first)."""
    entries = [(f.score, i, f.tokens) for i, f in enumerate(finished)]
    entries += [(float(c), len(finished) + b, t) for b, (c, t) in enumerate(zip(cum, tokens))]
    entries.sort(key=lambda e: (-e[0], e[1]))
    return [(np.float32(sc), toks) for sc, _, toks in entries]


def beam_search(prompt_k, prompt_v, prompt_cu, model, W, n_gen, eos, row_lse_for=None, scale=None):
    """Run the loop. prompt_k/v: packed prompt K/V [T_p, Nkv, D] (bf16 bits or tensors), prompt_cu [R+1].
    model(s) returns the step's synthetic model outputs: s = 0 -> {"logits": [R, 1, V]};
    s >= 1 -> {"q": [R, W, Nq, D], "k": [R, W, Nkv, D], "v": [R, W, Nkv, D], "logits": [R, W, V]}.
    row_lse_for(s) may return a [R, W_in] fp32 row log-sum-exp to select with (None: the oracle's own).
    Returns (list of StepRecord, final ranking per request)."""
    pk, pv = _bits(prompt_k), _bits(prompt_v)
    cu = np.asarray(prompt_cu, np.int64)
    R = len(cu) - 1
    nkv, d = pk.shape[1], pk.shape[2]
    # explicit per-beam K/V: at step 0 every request has one hypothesis (the prompt)
    full_k = [[pk[cu[r]:cu[r + 1]].copy()] for r in range(R)]
    full_v = [[pv[cu[r]:cu[r + 1]].copy()] for r in range(R)]
    lp = [int(cu[r + 1] - cu[r]) for r in range(R)]
    hist = [[[]] for _ in range(R)]
    cum = None
    finished = [[] for _ in range(R)]
    records = []
    for s in range(n_gen):
        m = model(s)
        out = lse = None
        if s > 0:
            q = _bits(m["q"])
            kn, vn = _bits(m["k"]), _bits(m["v"])
            # the current token's K/V joins every beam's own sequence
            for r in range(R):
                for b in range(W):
                    full_k[r][b] = np.concatenate([full_k[r][b], kn[r, b][None]])
                    full_v[r][b] = np.concatenate([full_v[r][b], vn[r, b][None]])
            # attention of every beam over its own explicit sequence: each beam a "request" with one beam
            seqs_k = [full_k[r][b] for r in range(R) for b in range(W)]
            seqs_v = [full_v[r][b] for r in range(R) for b in range(W)]
            bcu = np.concatenate([[0], np.cumsum([x.shape[0] for x in seqs_k])]).astype(np.int32)
            empty = np.zeros((R * W, 1, 1, nkv, d), np.uint16)
            o, l_ = shared_prefix_decode_packed(q.reshape(R * W, 1, *q.shape[2:]), np.concatenate(seqs_k),
                                                np.concatenate(seqs_v), bcu, empty, empty, 0, scale)
            out, lse = o.reshape(R, W, *o.shape[2:]), l_.reshape(R, W, -1)
        logits = m["logits"]
        w_in = 1 if s == 0 else W
        given = row_lse_for(s) if row_lse_for is not None else None
        sel = beam_topk(logits, cum, 2 * W, 2 * W, row_lse=given)
        new_par = np.zeros((R, W), np.int32)
        new_cum = np.zeros((R, W), np.float32)
        new_hist, new_k, new_v = [], [], []
        for r in range(R):
            par, toks, c, fin = advance(sel["tokens"][r], sel["parents"][r], sel["scores"][r], W, eos, hist[r])
            new_par[r], new_cum[r] = par, c
            finished[r].extend(fin)
            new_hist.append(toks)
            new_k.append([full_k[r][p].copy() for p in par])
            new_v.append([full_v[r][p].copy() for p in par])
        hist, full_k, full_v, cum = new_hist, new_k, new_v, new_cum
        records.append(StepRecord(
            s=s, attn_out=out, attn_lse=lse, cand_tokens=sel["tokens"], cand_parents=sel["parents"],
            cand_scores=sel["scores"], row_lse=sel["row_lse"], parents=new_par, tokens=[list(h) for h in hist],
            cum=cum.copy(),
            suffix_k=[[full_k[r][b][lp[r]:] for b in range(W)] for r in range(R)],
            suffix_v=[[full_v[r][b][lp[r]:] for b in range(W)] for r in range(R)],
            finished=[list(f) for f in finished]))
        assert w_in == (1 if s == 0 else W)
    final = [final_ranking(finished[r], cum[r], hist[r]) for r in range(R)]
    return records, final
