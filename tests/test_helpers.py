"""The tolerance helpers of the GPU parity tests, checked on the CPU."""
import numpy as np
import pytest
import torch

from helpers import bf16_tolerance, check_bf16, f32_ulp_gap


@pytest.mark.parametrize("ref,tol", [(1.9, 1e-2), (2.0, 1e-2), (3.9, 1e-2), (-3.99, 1e-2),
                                     (4.0, 2.0 ** -5), (-4.0, 2.0 ** -5), (7.9, 2.0 ** -5), (8.0, 2.0 ** -4),
                                     (0.0, 1e-2)])
def test_bf16_tolerance_widens_only_from_4(ref, tol):
    assert bf16_tolerance(np.array([ref]))[0] == tol


def test_check_bf16_bound_in_2_to_4():
    # |ref| in [2, 4): an error of 0.0156 (one bf16 ulp there) must fail, 0.0099 must pass
    ref = np.array([2.5, -3.5])
    check_bf16(torch.tensor([2.5 + 0.0099, -3.5 - 0.0099]), ref, "ok")
    with pytest.raises(AssertionError):
        check_bf16(torch.tensor([2.5 + 0.0156, -3.5]), ref, "too far")
    # at |ref| >= 4, one ulp (1/32) is allowed, two are not
    check_bf16(torch.tensor([4.0 + 1 / 32]), np.array([4.0]), "one ulp")
    with pytest.raises(AssertionError):
        check_bf16(torch.tensor([4.0 + 2 / 32]), np.array([4.0]), "two ulp")


def test_f32_ulp_gap():
    one = np.float32(1.0)
    assert f32_ulp_gap(one, np.nextafter(one, np.float32(2))) == 1
    assert f32_ulp_gap(np.float32(-0.0), np.float32(0.0)) == 0
    tiny = np.float32(np.finfo(np.float32).smallest_subnormal)
    assert f32_ulp_gap(-tiny, tiny) == 2
    x = np.float32(-20.5)
    y = x
    for _ in range(4):
        y = np.nextafter(y, np.float32(0))
    assert f32_ulp_gap(x, y) == 4
    from helpers import f32_ulp
    assert f32_ulp(np.float32(1.0)) == 2.0 ** -23 and f32_ulp(np.float32(-12.0)) == 2.0 ** -20


def test_cut_gap_on_oracle_runs_with_nudged_lse():
    """The top-K cut check, on two oracle runs whose row log-sum-exps differ by 1 and by 64 fp32 ulps: the
    first differs from the reference only at the cut (gap <= 4 ulp), the second is caught."""
    import oracle
    import workloads as wl
    from helpers import CUT_GAP_ULP, cut_gap

    # every beam of a request has the same logits and cumulative score: candidates tie across beams, so a
    # small change of some rows' log-sum-exp moves which beams' candidates make the cut
    x = wl.make_logits(2, 1, 3000, 3.0, seed=31).expand(2, 40, 3000).contiguous()
    cum = np.full((2, 40), -4.0, np.float32)
    ref = oracle.beam_topk(x, cum, 80, 40)
    seen = {}
    for nudge in (1, 64):
        lse = ref["row_lse"].copy()
        for _ in range(nudge):
            lse[:, ::2] = np.nextafter(lse[:, ::2], np.float32(np.inf))
        got = oracle.beam_topk(x, cum, 80, 40, row_lse=lse)
        res = []
        for i in range(2):
            if not np.array_equal(got["parents"][i], ref["parents"][i]) or \
                    not np.array_equal(got["tokens"][i], ref["tokens"][i]):
                res.append(cut_gap(got, ref, i, 80, 40))
        seen[nudge] = res
    assert seen[1] and all(g <= CUT_GAP_ULP and d <= CUT_GAP_ULP for g, d in seen[1])
    assert seen[64] and any(g > CUT_GAP_ULP or d > CUT_GAP_ULP for g, d in seen[64])
