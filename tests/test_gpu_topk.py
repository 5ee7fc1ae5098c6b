"""Two-stage beam top-K on the GPU against the oracle.

Stage-1 token ids depend only on the bf16 logits and must match bit for bit.
Scores depend on each row's fp32 log-sum-exp; the GPU's must be within 1e-5 of
the oracle's (fp64, rounded to fp32). Where that floating-point value decides
the integer results, both sides decide from the same value: the oracle run
with the GPU's row log-sum-exp must match every output bit for bit. Against
the oracle's own log-sum-exp, a request may differ only where a row's GPU value
differs from the oracle's fp32 value, and then only at the cut: every candidate
that one side selects and the other does not must score within 4 fp32 ulp of
the oracle's k_global-th score (and every candidate's GPU score within 4 ulp of
its oracle score), ulps taken at the larger of the score's and the row
log-sum-exp's magnitude (the score inherits the log-sum-exp's rounding). The GPU result must also be exactly the (-score, flat index)
top-k of the GPU's own stage-1 scores. The number of differing requests and the
largest gap at the cut are printed.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import CUT_GAP_ULP, cut_gap, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def bga():
    import attention_bga_packed_amd as m
    return m


def self_consistent(res, i, k_local, k_global):
    """GPU stage 2 is the exact top-k of the GPU's own stage-1 scores."""
    sc = res["local_scores"][i].cpu().numpy()
    w_in = sc.shape[0]
    f = np.arange(w_in * k_local)
    order = np.lexsort((f, -sc.ravel()))[:k_global]
    assert np.array_equal(res["parents"][i].cpu().numpy(), order // k_local)
    assert np.array_equal(res["scores"][i].cpu().numpy(), sc.ravel()[order])


def run_and_check(x, cum, k_local, k_global, name):
    say(f"[topk] {name} R={x.shape[0]} W_in={x.shape[1]} V={x.shape[2]} k_local={k_local} k_global={k_global}")
    xd = x.to(DEV)
    cd = None if cum is None else torch.from_numpy(cum).to(DEV)
    res = bga().beam_topk(xd, cd, k_local, k_global, want_local=True, want_lse=True)
    torch.cuda.synchronize()
    ref = oracle.beam_topk(x.cpu(), cum, k_local, k_global)
    assert np.array_equal(res["local_tokens"].cpu().numpy(), ref["local_tokens"]), "stage-1 ids differ"
    glse = res["row_lse"].cpu().numpy()
    lerr = np.abs(glse.astype(np.float64) - ref["row_lse64"])
    assert lerr.max() <= 1e-5, f"row lse error {lerr.max():.3e}"
    lse_diff = glse != ref["row_lse"]
    # scores are cum + (x - lse) in fp32 from the GPU's own lse
    xs = x.float().cpu().numpy()
    lt = res["local_tokens"].cpu().numpy()
    c = np.zeros(x.shape[:2], np.float32) if cum is None else cum
    lp = np.take_along_axis(xs, lt, axis=2) - glse[:, :, None]
    assert np.array_equal(res["local_scores"].cpu().numpy(), c[:, :, None] + lp), "stage-1 scores"
    # where floating point decides the selection, both sides decide from the same
    # fp32 row log-sum-exp (the kernel's): then everything must match bit for bit
    same_lse = oracle.beam_topk(x.cpu(), cum, k_local, k_global, row_lse=glse)
    for key in ("local_tokens", "local_scores", "tokens", "parents", "scores"):
        assert np.array_equal(res[key].cpu().numpy(), same_lse[key]), f"{key} differ given the same row lse"
    n_mismatch, worst_gap, worst_drift = 0, 0, 0
    for i in range(x.shape[0]):
        same = (np.array_equal(res["tokens"][i].cpu().numpy(), ref["tokens"][i])
                and np.array_equal(res["parents"][i].cpu().numpy(), ref["parents"][i])
                and np.array_equal(res["scores"][i].cpu().numpy(), ref["scores"][i]))
        if not same:
            n_mismatch += 1
            assert lse_diff[i].any(), f"request {i}: selection differs with identical row lse"
            gap, drift = cut_gap({k: t.cpu().numpy() for k, t in res.items()}, ref, i, k_local, k_global)
            assert drift <= CUT_GAP_ULP, f"request {i}: a candidate's GPU score is {drift:.2f} ulp from the oracle's"
            assert gap <= CUT_GAP_ULP, f"request {i}: a candidate {gap:.2f} ulp from the cut is selected differently"
            worst_gap, worst_drift = max(worst_gap, gap), max(worst_drift, drift)
        self_consistent(res, i, k_local, k_global)
    say(f"    rows with lse != oracle fp32: {int(lse_diff.sum())}/{lse_diff.size}; max |lse err| {lerr.max():.2e};"
        f" requests differing from the oracle's own lse: {n_mismatch}/{x.shape[0]}"
        f" (largest gap at the cut {worst_gap:.2f} ulp, largest score drift {worst_drift:.2f} ulp)")
    return res, ref


@pytest.mark.parametrize("v,std", [(1000, 3.0), (4096, 1.0), (333, 3.0), (64, 0.5)])
def test_small_random(v, std):
    x = wl.make_logits(3, 5, v, std, seed=v)
    cum = (np.random.default_rng(v).standard_normal((3, 5)) * 2 - 5).astype(np.float32)
    run_and_check(x, cum, min(10, v), 5, f"random V={v}")


def test_first_step_single_beam_no_cum():
    x = wl.make_logits(4, 1, 5000, 3.0, seed=1)
    run_and_check(x, None, 16, 8, "first step")


def test_heavy_ties():
    g = torch.Generator().manual_seed(3)
    x = torch.randint(-4, 5, (2, 6, 3000), generator=g).to(torch.bfloat16)
    cum = np.array([[0, 0, -1, 0, -1, 0], [-2] * 6], np.float32)
    for kl, kg in [(12, 6), (64, 64), (400, 100)]:
        run_and_check(x, cum, kl, kg, f"ties kl={kl} kg={kg}")


def test_all_equal_and_more_ties_than_fit():
    x = torch.full((1, 3, 20000), 0.75, dtype=torch.bfloat16)
    x[0, 1, 5] = 2.0
    run_and_check(x, np.zeros((1, 3), np.float32), 8, 5, "all equal")
    x = torch.zeros((1, 2, 9000), dtype=torch.bfloat16)
    x[0, :, ::3] = -0.0
    run_and_check(x, None, 1000, 1000, "zeros with -0")


def test_k_local_equals_vocab():
    x = wl.make_logits(2, 3, 256, 2.0, seed=4)
    run_and_check(x, None, 256, 7, "k_local = V")


def test_wide_beams_short_vocab():
    x = wl.make_logits(2, 400, 2048, 3.0, seed=6)
    cum = (np.random.default_rng(6).standard_normal((2, 400)) - 3).astype(np.float32)
    run_and_check(x, cum, 800, 400, "W=400 V=2048")
    run_and_check(x, cum, 800, 800, "W=400 V=2048 k_global=2W")


def test_long_beam_config_full():
    cfg = wl.CONFIGS["long_beam"]
    x = wl.make_logits(cfg["r"], cfg["w"], cfg["vocab"], cfg["logit_std"], seed=cfg["seed"] + 1, device=DEV).cpu()
    cum = (np.random.default_rng(0).standard_normal((cfg["r"], cfg["w"])) * 3 - 20).astype(np.float32)
    run_and_check(x, cum, 2 * cfg["w"], cfg["w"], "long_beam")


def test_caps_512_beams_k_1024():
    """BGA_MAX_BEAMS source beams, k_local = k_global = BGA_MAX_K (2W global candidates at W = 512)."""
    x = wl.make_logits(1, 512, 151936, 3.0, seed=512, device=DEV).cpu()
    cum = (np.random.default_rng(512).standard_normal((1, 512)) - 10).astype(np.float32)
    run_and_check(x, cum, 1024, 1024, "caps W=512 k=1024")


def test_determinism():
    x = wl.make_logits(2, 50, 30000, 3.0, seed=9).to(DEV)
    r1 = bga().beam_topk(x, None, 100, 50, want_local=True, want_lse=True)
    r2 = bga().beam_topk(x, None, 100, 50, want_local=True, want_lse=True)
    for key in r1:
        assert torch.equal(r1[key], r2[key]), key


def strided_sample_chunks(vocab, n_sample_chunks=512):
    """The 8-logit chunks an evenly strided sample of a row visits (chunk i * n / s)."""
    n = (vocab + 7) // 8
    s = min(n, n_sample_chunks)
    return np.unique((np.arange(s) * n) // s)


def test_sample_that_misleads_the_threshold():
    """Rows whose sampled chunks are all large: the sampled cut admits fewer
    than k_local keys, so stage 1 must fall back to an exact select over the
    whole row (and still match the oracle)."""
    v = 20000
    x = wl.make_logits(2, 3, v, 1.0, seed=21).float()
    for c in strided_sample_chunks(v):
        x[:, :, c * 8:(c + 1) * 8] += 6.0
    x = x.to(torch.bfloat16)
    run_and_check(x, None, 200, 6, "sample misleads")


def test_candidates_spanning_many_keys():
    """Logits spread over many binades: the keys at or above the cut span more
    than the counting sort's bins, which takes the general path."""
    g = torch.Generator().manual_seed(22)
    mag = torch.exp2(torch.rand((2, 4, 10000), generator=g) * 123 - 120)   # |x| <= 8: the lse stays O(1)
    sign = torch.where(torch.rand((2, 4, 10000), generator=g) < 0.5, -1.0, 1.0)
    x = (mag * sign).to(torch.bfloat16)
    run_and_check(x, None, 300, 8, "wide key range")


def test_ties_beyond_the_candidate_list():
    """Few distinct values in a long row: the keys at or above the cut exceed
    the candidate list, and ties at the cut are resolved by lower id."""
    g = torch.Generator().manual_seed(23)
    x = torch.randint(-2, 3, (2, 3, 30000), generator=g).to(torch.bfloat16)
    run_and_check(x, np.zeros((2, 3), np.float32), 64, 20, "ties beyond list")


def test_one_beam_dominates_the_request():
    """One beam's cumulative score dwarfs the others: all global winners come
    from it, deeper than the first entries stage 2 loads up front."""
    x = wl.make_logits(2, 50, 5000, 3.0, seed=24)
    cum = np.zeros((2, 50), np.float32)
    cum[:, 7] = 100.0
    run_and_check(x, cum, 100, 50, "dominant beam")
