"""Pins for the GRPO/DAPO token-loss oracle: closed forms, a hand-worked branch
table (tests/golden/grpo_branches.json) and finite differences."""
import json
import math
import os

import numpy as np
import pytest

from oracle import grpo
from oracle import grpo as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bernoulli_group_closed_form():
    # k successes in a group of 8, unbiased std: A_success = (1 - k/8) / sqrt(k (8 - k) / 56)
    for k in range(1, 8):
        r = np.array([1.0] * k + [0.0] * (8 - k))
        A = grpo.advantages(r, 8, grpo.Params(adv_eps=0.0))
        sd = math.sqrt(k * (8 - k) / 56.0)
        assert A[0] == pytest.approx((1 - k / 8) / sd, rel=1e-14)
        assert A[-1] == pytest.approx((-k / 8) / sd, rel=1e-14)
    for c in (0.0, 1.0):                       # a constant group has no signal
        assert np.all(grpo.advantages(np.full(8, c), 8) == 0.0)


@pytest.mark.parametrize("c", [0.0, 1.0, 0.1, -3.7])
@pytest.mark.parametrize("prm", [grpo.Params(adv_eps=0.0), grpo.Params(),
                                 grpo.Params(adv_eps=0.0, std_ddof=0),
                                 grpo.Params(normalize_std=False),
                                 grpo.Params(adv_eps=0.0, baseline="length")])
def test_constant_group_is_zero_in_every_mode(c, prm):
    """A constant group's advantages are exactly 0, also with adv_eps = 0
    (no 0/0), with a length-weighted baseline (no rounding residue) and beside
    a group that does vary; the loss of such a batch stays finite."""
    r = np.concatenate([np.full(8, c), [1, 0, 0, 1, 1, 0, 1, 1]]).astype(np.float32)
    lengths = np.arange(3, 19)
    A = grpo.advantages(r, 8, prm, lengths=lengths)
    assert np.all(A[:8] == 0.0) and np.all(np.isfinite(A))
    assert np.all(A[8:] != 0.0)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    lp = np.linspace(-3, -0.1, cu[-1])
    out = grpo.token_loss(lp, lp - 0.01, lp, cu, A, prm)
    assert np.isfinite(out.loss) and np.all(np.isfinite(out.grad))
    assert np.all(out.grad[:cu[8]] == 0.0)     # rho != 1 but A = 0 and k3' = 0 at ref = new


def test_on_policy_identity():
    rng = np.random.default_rng(1)
    lengths = rng.integers(1, 30, size=16)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    lp = rng.normal(-2, 1, cu[-1])
    A = grpo.advantages(rng.integers(0, 2, 16).astype(float), 8)
    r = grpo.token_loss(lp, lp, lp, cu, A)
    # rho = 1, k3 = 0: L = -sum_j L_j A_j / T_tot
    assert r.loss == pytest.approx(-(lengths * A).sum() / cu[-1], rel=1e-12, abs=1e-15)
    assert r.metrics[1] == 0.0 and r.metrics[2] == 0.0 and r.metrics[3] == 1.0
    # equal lengths: advantages sum to zero per group, so the loss is zero
    cu2 = np.arange(17) * 5
    r2 = grpo.token_loss(lp[:80], lp[:80], lp[:80], cu2, A)
    assert abs(r2.loss) < 1e-15


def test_k3_closed_form():
    cu = np.array([0, 3])
    lp_new = np.zeros(3)
    lp_ref = np.array([0.0, math.log(2.0), -1.0])
    r = grpo.token_loss(lp_new, lp_new, lp_ref, cu, np.zeros(1), grpo.Params(kl_coef=1.0))
    expect = [0.0, 1.0 - math.log(2.0), math.exp(-1.0)]
    np.testing.assert_allclose(r.token_loss, expect, rtol=1e-14, atol=1e-16)


def test_branch_table():
    """Hand-worked surrogate values and gradients (C=2, eps 0.2/0.28, beta=0)."""
    with open(os.path.join(GOLDEN, "grpo_branches.json")) as f:
        table = json.load(f)["cases"]
    prm = grpo.Params(kl_coef=0.0)
    for case in table:
        rho, A = case["rho"], case["A"]
        cu = np.array([0, 1])
        r = grpo.token_loss(np.array([math.log(rho)]), np.zeros(1), np.array([math.log(rho)]),
                            cu, np.array([A]), prm)
        assert r.token_loss[0] == pytest.approx(case["loss"], rel=1e-12, abs=1e-15), case
        assert r.grad[0] == pytest.approx(case["grad"], rel=1e-12, abs=1e-15), case
        assert int(r.flags[0]) == case["flags"], case


def test_gradient_finite_differences():
    rng = np.random.default_rng(2)
    lengths = rng.integers(1, 12, size=8)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    n = cu[-1]
    lp_new = rng.normal(-1.5, 1.0, n)
    lp_old = lp_new + rng.normal(0, 0.4, n)
    lp_ref = lp_new + rng.normal(0, 0.3, n)
    A = grpo.advantages(rng.integers(0, 2, 8).astype(float), 4)
    base = grpo.token_loss(lp_new, lp_old, lp_ref, cu, A)
    eps = 1e-7
    for t in range(n):
        if base.near_branch[t]:
            continue
        lp_p, lp_m = lp_new.copy(), lp_new.copy()
        lp_p[t] += eps
        lp_m[t] -= eps
        num = (grpo.token_loss(lp_p, lp_old, lp_ref, cu, A).loss
               - grpo.token_loss(lp_m, lp_old, lp_ref, cu, A).loss) / (2 * eps)
        assert base.grad[t] == pytest.approx(num, rel=1e-5, abs=1e-9)


def test_empty_batch():
    r = grpo.token_loss(np.zeros(0), np.zeros(0), np.zeros(0), np.array([0, 0, 0]), np.zeros(2))
    assert r.loss == 0.0 and r.grad.size == 0


# ------------------------------------------------------------ loss variants

def _one(lpn, lpo, A, **kw):
    """One response of one token (reference logprob = new: no KL)."""
    prm = G.Params(kl_coef=0.0, **kw)
    return G.token_loss(np.array([lpn]), np.array([lpo]), np.array([lpn]), np.array([0, 1]),
                        np.array([A]), prm)


def test_ipo_mask_closed_form():
    # pi_old = 0.5: pi_new 0.75 moved 0.25 (kept), 0.85 moved 0.35 (masked)
    lpo = np.log(0.5)
    r = _one(np.log(0.75), lpo, 2.0, loss_type="ipo", ipo_eps=0.3, tis_cap=10.0)
    assert r.loss == pytest.approx(-1.5 * 2.0) and r.grad[0] == pytest.approx(-2.0 * 1.5)
    assert r.flags[0] == 0
    r = _one(np.log(0.85), lpo, 2.0, loss_type="ipo", ipo_eps=0.3, tis_cap=10.0)
    assert r.loss == 0.0 and r.grad[0] == 0.0 and r.flags[0] == G.FLAG_CLIP
    # the mask ignores the sign of the advantage and is double-sided
    r = _one(np.log(0.15), lpo, -1.0, loss_type="ipo", ipo_eps=0.3, tis_cap=10.0)
    assert r.grad[0] == 0.0 and r.flags[0] == G.FLAG_CLIP


def test_icepop_band_closed_form():
    for rho, kept in ((0.4, False), (0.6, True), (1.9, True), (2.5, False)):
        r = _one(np.log(rho), 0.0, 1.0, loss_type="icepop", icepop_lo=0.5, icepop_hi=2.0,
                 tis_cap=10.0)
        assert (r.flags[0] == 0) == kept
        assert r.grad[0] == pytest.approx(-rho if kept else 0.0, rel=1e-12)
        assert r.loss == pytest.approx(-rho if kept else 0.0, rel=1e-12)


def test_cispo_closed_form():
    # the weight is the clipped ratio, held constant: loss -w A lp_new, gradient -w A
    for rho, w in ((0.5, 0.8), (1.1, 1.1), (1.6, 1.28)):
        lpn = np.log(rho) - 0.7
        r = _one(lpn, -0.7, 3.0, loss_type="cispo", tis_cap=10.0)
        assert r.grad[0] == pytest.approx(-w * 3.0, rel=1e-12)
        assert r.loss == pytest.approx(-w * 3.0 * lpn, rel=1e-12)
        assert (r.flags[0] == G.FLAG_CLIP) == (w != rho)


def test_mis_normalises_the_ratios():
    rng = np.random.default_rng(11)
    T = 50
    lpo = rng.normal(-1, 0.5, T)
    lpn = lpo + 0.3                               # every ratio e^0.3: normalised to 1
    cu = np.array([0, 20, 50])
    r = G.token_loss(lpn, lpo, lpn, cu, np.array([1.5, -0.5]),
                     G.Params(kl_coef=0.0, correction="mis"), group_size=2)
    A = np.repeat([1.5, -0.5], [20, 30])
    np.testing.assert_allclose(r.token_loss, -A, rtol=1e-12)
    np.testing.assert_allclose(r.grad, -A / T, rtol=1e-12)
    assert not r.flags.any()


def test_aggregation_and_filtering_weights():
    cu = np.array([0, 1, 4, 6, 8])                # lengths 1, 3 | 2, 2
    A = np.array([1.0, -1.0, 0.0, 0.0])
    w = G.weights(cu, A, 2, G.Params(aggregation="prompt_mean"))
    np.testing.assert_allclose(w, [1 / 8] * 4 + [1 / 8] * 4)
    w = G.weights(cu, A, 2, G.Params(aggregation="prompt_mean", filter_zero_adv=True))
    np.testing.assert_allclose(w, [1 / 4] * 4 + [0.0] * 4)
    w = G.weights(cu, A, 2, G.Params(filter_zero_adv=True))
    np.testing.assert_allclose(w, [1 / 4] * 4 + [0.0] * 4)
    w = G.weights(cu, np.zeros(4), 2, G.Params(filter_zero_adv=True))
    assert not w.any()
    # prompt mean = mean over groups of each group's token mean
    rng = np.random.default_rng(12)
    lpn, lpo = rng.normal(-1, 0.3, 8), rng.normal(-1, 0.3, 8)
    prm = G.Params(aggregation="prompt_mean")
    r = G.token_loss(lpn, lpo, lpn, cu, np.array([1.0, -1.0, 0.5, -0.5]), prm, group_size=2)
    assert r.loss == pytest.approx(0.5 * (r.token_loss[:4].mean() + r.token_loss[4:].mean()))


def test_length_weighted_baseline():
    prm = G.Params(baseline="length", normalize_std=False)
    a = G.advantages(np.array([1.0, 0.0, 1.0, 1.0]), 2, prm, lengths=[3, 1, 5, 5])
    np.testing.assert_allclose(a, [0.25, -0.75, 0.0, 0.0])
    prm = G.Params(baseline="length")
    a = G.advantages(np.array([1.0, 0.0]), 2, prm, lengths=[1, 1])   # equal lengths: the mean
    np.testing.assert_allclose(a, G.advantages(np.array([1.0, 0.0]), 2, G.Params()))


@pytest.mark.parametrize("loss_type,agg,filt", [("dapo", "prompt_mean", True),
                                                ("ipo", "token_mean", False),
                                                ("icepop", "prompt_mean", False),
                                                ("dapo", "token_mean", True)])
def test_variant_gradients_by_finite_differences(loss_type, agg, filt):
    rng = np.random.default_rng(13)
    cu = np.array([0, 5, 9, 12, 20])
    T = 20
    lpo = rng.normal(-1.0, 0.4, T)
    lpn = lpo + rng.normal(0, 0.3, T)
    lpr = lpn + rng.normal(0, 0.1, T)
    A = np.array([0.7, 0.0, -1.1, 0.4])
    prm = G.Params(loss_type=loss_type, aggregation=agg, filter_zero_adv=filt, tis_cap=1.5,
                   icepop_lo=0.7, icepop_hi=1.3, ipo_eps=0.15)
    r = G.token_loss(lpn, lpo, lpr, cu, A, prm, group_size=2)
    eps = 1e-7
    for t in range(T):
        if r.near_branch[t]:
            continue
        up, dn = lpn.copy(), lpn.copy()
        up[t] += eps
        dn[t] -= eps
        num = (G.token_loss(up, lpo, lpr, cu, A, prm, 2).loss -
               G.token_loss(dn, lpo, lpr, cu, A, prm, 2).loss) / (2 * eps)
        assert r.grad[t] == pytest.approx(num, rel=1e-5, abs=1e-9), t


def test_detached_tis_form_closed_form():
    # the weight min(rho, C) is a constant and the surrogate's own ratio is 1:
    # loss -w A and gradient -w A, whether or not the cap binds
    for rho, w in ((0.7, 0.7), (1.9, 1.9), (3.0, 2.0)):
        r = _one(np.log(rho) - 1.0, -1.0, -1.5, loss_type="tis_pg", tis_cap=2.0)
        assert r.loss == pytest.approx(w * 1.5, rel=1e-12)
        assert r.grad[0] == pytest.approx(w * 1.5, rel=1e-12)
        assert r.flags[0] == (G.FLAG_TIS if rho > 2.0 else 0)
