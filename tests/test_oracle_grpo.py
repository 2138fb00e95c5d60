"""Pins for the GRPO/DAPO token-loss oracle: closed forms, a hand-worked branch
table (tests/golden/grpo_branches.json) and finite differences."""
import json
import math
import os

import numpy as np
import pytest

from oracle import grpo

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
