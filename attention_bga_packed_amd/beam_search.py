"""Fixed-depth beam search over the library's calls (argument marshalling and
the fixed call sequence only; every step runs in the HIP kernels).

The article's bounded generation (section 2.3) runs a loop whose control flow is
fixed at deployment: prompt prefill -> first-step candidate initialisation ->
(N_gen - 1) x [decode -> per-beam candidate selection -> cumulative score merge
-> parent index update -> token and suffix K/V reorder] -> final candidates and
scores; the state's capacities are fixed too, only its contents depend on the
model's outputs. This class holds that fixed-capacity state on the device and
issues, per step, the same sequence of calls:

    start(logits of the prompts' last tokens)       bga_beam_topk (W_in = 1) -> bga_beam_advance
    decode(q, k_new, v_new)                         bga_suffix_append -> bga_shared_prefix_decode_packed
    select(logits)                                  bga_beam_topk (2W / 2W) -> bga_beam_advance -> bga_suffix_reorder
    finish()                                        bga_beam_finalize

The model between decode and select (its outputs are the query, the new
token's K/V and the logits) is not part of this path; callers pass its outputs.
The prompts' K/V are the packed prefill's K/V, used as the shared prefix as they
are (prompt_cu gives each request's rows).

Every call works in the state allocated here (the final ranking's buffers
after the first finish()), clears nothing and never waits on the host, so once
a loop has run, a whole loop can be captured into a HIP graph
(torch.cuda.graph) and replayed; a replay reads the model outputs from the
tensors the capture saw.
"""
from __future__ import annotations

import math

import torch

from . import _binding as B


class BeamSearch:
    def __init__(self, num_requests: int, beam_width: int, n_gen: int, vocab: int, num_q_heads: int,
                 num_kv_heads: int, head_dim: int, stop_token: int, device, softmax_scale=None):
        R, W = num_requests, beam_width
        self.R, self.W, self.n_gen, self.V = R, W, n_gen, vocab
        self.nq, self.nkv, self.d = num_q_heads, num_kv_heads, head_dim
        self.stop = stop_token
        self.scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(head_dim)
        dev = torch.device(device)
        i32, f32, bf = torch.int32, torch.float32, torch.bfloat16
        cap = max(1, n_gen - 1)
        self.suffix = [(torch.zeros((R, W, cap, num_kv_heads, head_dim), dtype=bf, device=dev),
                        torch.zeros((R, W, cap, num_kv_heads, head_dim), dtype=bf, device=dev)) for _ in range(2)]
        self.tokens = [torch.zeros((R, W, n_gen), dtype=i32, device=dev) for _ in range(2)]
        self.tokens0 = torch.zeros((R, 1, n_gen), dtype=i32, device=dev)   # the prompt's (empty) history
        self.cum = [torch.zeros((R, W), dtype=f32, device=dev) for _ in range(2)]
        self.parents = torch.zeros((R, W), dtype=i32, device=dev)
        self.cand = {"tokens": torch.zeros((R, 2 * W), dtype=i32, device=dev),
                     "parents": torch.zeros((R, 2 * W), dtype=i32, device=dev),
                     "scores": torch.zeros((R, 2 * W), dtype=f32, device=dev),
                     "row_lse": torch.zeros((R, W), dtype=f32, device=dev)}
        self.cand0 = {k: v for k, v in self.cand.items() if k != "row_lse"}
        self.cand0["row_lse"] = torch.zeros((R, 1), dtype=f32, device=dev)
        P = W * n_gen
        self.pool = {"scores": torch.zeros((R, P), dtype=f32, device=dev),
                     "lengths": torch.zeros((R, P), dtype=i32, device=dev),
                     "tokens": torch.zeros((R, P, n_gen), dtype=i32, device=dev),
                     "count": torch.zeros((R,), dtype=i32, device=dev)}
        self.ws = torch.empty(max(B.beam_topk_workspace_size(R, W, vocab, 2 * W, 2 * W), 1), dtype=torch.uint8,
                              device=dev)
        self.out = torch.empty((R, W, num_q_heads, head_dim), dtype=bf, device=dev)
        self.lse = torch.empty((R, W, num_q_heads), dtype=f32, device=dev)
        self.final = None
        self.cur = 0
        self.s = 0
        self.prompt = None

    def start(self, prompt_k, prompt_v, prompt_cu, logits0):
        """First-step initialisation from the prompts' last-token logits [R, 1, V]; prompt K/V [T_p, Nkv, D]
        (the packed prefill's), prompt_cu [R + 1] int32 on the device."""
        self.prompt = (prompt_k, prompt_v, prompt_cu)
        self.cur, self.s = 0, 0
        B.beam_topk(logits0, None, 2 * self.W, 2 * self.W, workspace=self.ws, out=self.cand0)
        B.beam_advance(self.cand0["tokens"], self.cand0["parents"], self.cand0["scores"], self.W, self.stop, 0,
                       self.tokens0, self.tokens[0], self.parents, self.cum[0], self.pool)
        self.s = 1
        return self.cand0

    def decode(self, q, k_new, v_new):
        """Decode step s: the current tokens' K/V into suffix position s - 1, then attention over
        [prompt; suffix 0..s-1]. Returns (out [R, W, Nq, D], lse [R, W, Nq])."""
        s = self.s
        if not 1 <= s < self.n_gen:
            raise RuntimeError(f"decode at step {s} of {self.n_gen}")
        sk, sv = self.suffix[self.cur]
        B.suffix_append(k_new, v_new, sk, sv, s - 1)
        pk, pv, pcu = self.prompt
        return B.shared_prefix_decode_packed(q, pk, pv, pcu, sk, sv, s, self.scale, out=self.out, lse=self.lse)

    def select(self, logits):
        """Candidate selection and state update of step s from logits [R, W, V]."""
        s, c = self.s, self.cur
        B.beam_topk(logits, self.cum[c], 2 * self.W, 2 * self.W, workspace=self.ws, out=self.cand)
        B.beam_advance(self.cand["tokens"], self.cand["parents"], self.cand["scores"], self.W, self.stop, s,
                       self.tokens[c], self.tokens[1 - c], self.parents, self.cum[1 - c], self.pool)
        sk, sv = self.suffix[c]
        nk, nv = self.suffix[1 - c]
        B.suffix_reorder(sk, sv, self.parents, s, dst_k=nk, dst_v=nv)
        self.cur, self.s = 1 - c, s + 1
        return self.cand

    @property
    def state(self):
        """The current beams: tokens [R, W, n_gen] (first s valid), cumulative scores [R, W], suffix K/V."""
        c = self.cur
        return {"tokens": self.tokens[c], "cum": self.cum[c], "suffix_k": self.suffix[c][0],
                "suffix_v": self.suffix[c][1], "parents": self.parents, "pool": self.pool, "generated": self.s}

    def finish(self):
        """Final candidates and scores: finished hypotheses and the beams, ranked best first."""
        c = self.cur
        self.final = B.beam_finalize(self.pool, self.cum[c], self.tokens[c], self.s, out=self.final)
        return self.final
