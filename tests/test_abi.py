"""The C-ABI library on the host (no GPU needed): it loads, exports every symbol
include/bga.h declares, and rejects bad arguments with the documented status
before making any device call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def m():
    import attention_bga_packed_amd as mod
    return mod


def header_symbols():
    text = open(os.path.join(ROOT, "include", "bga.h")).read()
    return sorted(set(re.findall(r"\b(bga_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header(m):
    syms = header_symbols()
    assert syms == sorted(m.EXPORTS)
    raw = ctypes.CDLL(m.LIB_PATH)
    for s in syms:
        assert hasattr(raw, s), s


def test_status_strings(m):
    for code in range(9):
        s = m.lib.bga_status_string(code).decode()
        assert s.startswith("BGA_")
        assert s.split(":")[0] == m._binding.STATUS_NAMES[code]
    assert m.lib.bga_last_hip_error() == 0
    assert m.lib.bga_last_violations() == 0
    assert m.lib.bga_version() >= 200


def test_release_and_debug_builds():
    from attention_bga_packed_amd import _binding
    rel = _binding.load_library(_binding.RELEASE_LIB_PATH)
    dbg = _binding.load_library(_binding.DEBUG_LIB_PATH)
    assert rel.bga_debug_build() == 0 and dbg.bga_debug_build() == 1
    for s in header_symbols():
        assert hasattr(dbg, s), s


def header_caps():
    text = open(os.path.join(ROOT, "include", "bga.h")).read()
    return {k: int(v) for k, v in re.findall(r"#define (BGA_MAX_[A-Z]+) (\d+)", text)}


def test_caps_are_the_contract():
    # the article's bounds with headroom: <= 512 beams, <= 16 suffix tokens, sequences <= 8192 tokens
    assert header_caps() == {"BGA_MAX_GROUP": 16, "BGA_MAX_SEQLEN": 8192, "BGA_MAX_BEAMS": 512,
                             "BGA_MAX_SUFFIX": 16, "BGA_MAX_K": 1024, "BGA_MAX_VOCAB": 163840}


P = 0x10000  # a fake, 16-byte aligned "device" address: never dereferenced on these paths


def prefill(m, q=P, k=2 * P, v=3 * P, cu=4 * P, B=3, T=62, maxL=40, nq=4, nkv=2, d=64, scale=0.125,
            out=5 * P, lse=6 * P):
    return m.lib.bga_packed_gqa_prefill(q, k, v, cu, B, T, maxL, nq, nkv, d, scale, out, lse, None)


def test_prefill_errors(m):
    assert prefill(m, nq=5, nkv=2) == 2
    assert prefill(m, d=96) == 3
    assert prefill(m, nq=34, nkv=2) == 3          # group 17
    assert prefill(m, T=-1) == 2
    assert prefill(m, scale=0.0) == 2
    assert prefill(m, cu=None) == 1
    assert prefill(m, q=None) == 1
    assert prefill(m, out=None) == 1
    assert prefill(m, k=2 * P + 8) == 4
    assert prefill(m, lse=6 * P + 2) == 4
    assert prefill(m, out=P) == 6                 # out aliases q
    assert prefill(m, maxL=1 << 20) == 3
    assert prefill(m, maxL=8193) == 3
    assert prefill(m, maxL=0) == 2                # rows exist but no sequence may hold one
    assert prefill(m, B=0) == 2
    assert prefill(m, T=0) == 0                   # nothing to do, nothing launched
    assert prefill(m, T=0, B=0, maxL=0) == 0


def decode(m, q=P, pk=2 * P, pv=3 * P, sk=4 * P, sv=5 * P, R=2, W=4, Lp=8, Ls=2, cap=3, nq=4, nkv=2, d=64,
           scale=0.125, out=6 * P, lse=7 * P):
    return m.lib.bga_shared_prefix_decode(q, pk, pv, sk, sv, R, W, Lp, Ls, cap, nq, nkv, d, scale, out, lse, None)


def test_decode_errors(m):
    assert decode(m, Ls=4, cap=3) == 2
    assert decode(m, Lp=0, Ls=0) == 2
    assert decode(m, W=2000) == 3
    assert decode(m, W=513) == 3
    assert decode(m, cap=100, Ls=1) == 3
    assert decode(m, cap=17, Ls=1) == 3
    assert decode(m, Lp=8193) == 3
    assert decode(m, d=80) == 3
    assert decode(m, sk=None) == 1
    assert decode(m, pk=None) == 1
    assert decode(m, q=P + 4) == 4
    assert decode(m, out=P) == 6
    assert decode(m, R=0) == 0


def reorder(m, sk=P, sv=2 * P, dk=3 * P, dv=4 * P, par=5 * P, st=None, dt=None, R=2, W=4, Ls=2, cap=3, nkv=2,
            d=64, nt=0, tc=0):
    return m.lib.bga_suffix_reorder(sk, sv, dk, dv, par, st, dt, R, W, Ls, cap, nkv, d, nt, tc, None)


def test_reorder_errors(m):
    assert reorder(m, Ls=4) == 2
    assert reorder(m, st=6 * P) == 1              # tokens: both or neither
    assert reorder(m, st=6 * P, dt=7 * P, nt=5, tc=4) == 2
    assert reorder(m, dk=P) == 6                  # dst overlaps src
    assert reorder(m, par=None) == 1
    assert reorder(m, dk=3 * P + 2) == 4
    assert reorder(m, W=513) == 3
    assert reorder(m, cap=17) == 3
    assert reorder(m, W=0) == 0


def topk(m, logits=P, cum=None, R=2, W=4, V=1000, kl=8, kg=4, tok=2 * P, par=3 * P, sc=4 * P, ws=8 * P,
         wsb=None):
    if wsb is None:
        wsb = m.beam_topk_workspace_size(R, W, V, kl, kg)
    return m.lib.bga_beam_topk(logits, cum, R, W, V, kl, kg, tok, par, sc, None, None, None, ws, wsb, None)


def test_topk_errors(m):
    assert m.beam_topk_workspace_size(2, 4, 1000, 8, 4) > 0
    assert m.beam_topk_workspace_size(2, 4, 1000, 2000, 4) == 0
    assert topk(m, kl=2000) == 2                  # k_local > V
    assert topk(m, kg=33) == 2                    # k_global > W * k_local
    assert topk(m, kl=1025, V=5000) == 3
    assert topk(m, V=200000) == 3
    assert topk(m, W=2000) == 3
    assert topk(m, W=513, kg=4) == 3
    assert topk(m, tok=None) == 1
    assert topk(m, wsb=16) == 5
    assert topk(m, ws=None) == 5
    assert topk(m, logits=P + 2) == 4
    assert topk(m, R=0) == 0


def test_topk_noalloc_errors(m):
    def na(R=2, W=4, V=1000, kl=8, kg=4, logits=P, tok=2 * P):
        return m.lib.bga_beam_topk_noalloc(logits, None, R, W, V, kl, kg, tok, 3 * P, 4 * P, None, None, None, None)
    assert na(kl=2000) == 2
    assert na(tok=None) == 1
    assert na(logits=P + 2) == 4
    assert na(R=0) == 0
    # the library's own workspace holds 24 MiB: 8 x 400 beams with k_local 800 fit, 8 x 512 x 1024 do not
    assert m.beam_topk_workspace_size(8, 400, 151936, 800, 400) <= 24 << 20
    assert na(R=8, W=512, V=151936, kl=1024, kg=1024) == 5


def test_decode_packed_errors(m):
    def dp(q=P, pk=2 * P, pv=3 * P, cu=8 * P, tp=20, sk=4 * P, sv=5 * P, R=2, W=4, Ls=2, cap=3, nq=4, nkv=2, d=64,
           out=6 * P, lse=7 * P):
        return m.lib.bga_shared_prefix_decode_packed(q, pk, pv, cu, tp, sk, sv, R, W, Ls, cap, nq, nkv, d, 0.125, out,
                                                     lse, None)
    assert dp(tp=-1) == 2
    assert dp(tp=0, Ls=0) == 2          # no key anywhere
    assert dp(Ls=4) == 2
    assert dp(W=513) == 3
    assert dp(cu=None) == 1
    assert dp(pk=None) == 1
    assert dp(cu=8 * P + 2) == 4
    assert dp(out=2 * P) == 6           # out overlaps the prompt K
    assert dp(R=0) == 0


def test_last_token_gather_errors(m):
    def g(src=P, cu=2 * P, B=3, T=10, rb=256, dst=3 * P):
        return m.lib.bga_last_token_gather(src, cu, B, T, rb, dst, None)
    assert g(rb=100) == 2               # not a multiple of 16
    assert g(rb=0) == 2
    assert g(B=-1) == 2
    assert g(cu=None) == 1
    assert g(dst=None) == 1
    assert g(src=P + 8) == 4
    assert g(dst=P + 16 * 5) == 6       # dst inside src
    assert g(B=0) == 0


def test_beam_state_update_errors(m):
    def adv(R=2, Win=4, W=4, step=1, tc=5, pc=8, ti=P, to=2 * P):
        return m.lib.bga_beam_advance(3 * P, 4 * P, 5 * P, R, Win, W, 7, step, ti, to, tc, 6 * P, 7 * P, 8 * P, 9 * P,
                                      10 * P, 11 * P, pc, None)
    assert adv(Win=5) == 2              # more source beams than beams
    assert adv(step=5) == 2             # no room for the new token
    assert adv(pc=0) == 2
    assert adv(W=513, Win=1) == 3
    assert adv(ti=None) == 1
    assert adv(to=P + 2) == 4
    assert adv(to=P) == 6               # new token lists over the old ones
    assert adv(R=0) == 0

    def app(R=2, W=4, pos=1, cap=3, nk=P, sk=2 * P):
        return m.lib.bga_suffix_append(nk, 3 * P, sk, 4 * P, R, W, pos, cap, 2, 64, None)
    assert app(pos=3) == 2
    assert app(cap=17, pos=1) == 3
    assert app(nk=None) == 1
    assert app(sk=2 * P + 4) == 4
    assert app(nk=2 * P) == 6
    assert app(W=0) == 0

    def fin(R=2, W=4, pc=8, ln=3, tc=5):
        return m.lib.bga_beam_finalize(P, 2 * P, 3 * P, 4 * P, pc, 5 * P, 6 * P, R, W, ln, tc, 7 * P, 8 * P, 9 * P,
                                       10 * P, None)
    assert fin(ln=6) == 2
    assert fin(ln=0) == 2
    assert fin(pc=8190) == 3            # more than 8192 entries to rank
    assert fin(R=0) == 0


def test_swiglu_quant_errors(m):
    def sq(x=P, T=4, I=64, c=2 * P, s=3 * P):
        return m.lib.bga_swiglu_quant_e4m3(x, T, I, c, s, None)
    assert sq(I=60) == 2
    assert sq(I=0) == 2
    assert sq(T=-1) == 2
    assert sq(I=16392) == 3
    assert sq(c=None) == 1
    assert sq(c=2 * P + 4) == 4
    assert sq(c=P + 8) == 6             # codes inside gate_up
    assert sq(T=0) == 0
