"""GPU parity of rlk_grpo_token_loss against the fp64 oracle on identical fp32
inputs: loss, metrics and dL/dlp_new within 1e-6 relative; per-token flags
exact except tokens whose ratio sits within 1e-6 of a branch point."""
import numpy as np
import pytest
import torch

import synth
from oracle import grpo as OG
import grpo_loss_rlk_amd as rlk

from gpu_util import f32_to_device, host

pytestmark = pytest.mark.gpu


def _inputs(seed, lengths, sd_old=0.05, sd_ref=0.1):
    rng = np.random.default_rng(seed)
    cu = synth.cu_seqlens(np.asarray(lengths))
    T = int(cu[-1])
    lp_new = rng.normal(-2.0, 1.5, T).astype(np.float32)
    lp_old = (lp_new + rng.normal(0, sd_old, T)).astype(np.float32)
    lp_ref = (lp_new + rng.normal(0, sd_ref, T)).astype(np.float32)
    return cu, lp_new, lp_old, lp_ref


def _compare(out, o, near):
    assert float(host(out["loss"])) == pytest.approx(o.loss, rel=1e-6, abs=1e-9)
    np.testing.assert_allclose(host(out["metrics"]), o.metrics, rtol=1e-6, atol=1e-9)
    g = host(out["grad"])
    keep = ~near
    np.testing.assert_allclose(g[keep], o.grad[keep], rtol=1e-6, atol=1e-12)
    np.testing.assert_allclose(host(out["token_loss"]), o.token_loss, rtol=1e-6, atol=1e-7)
    np.testing.assert_array_equal(host(out["token_flags"])[keep], o.flags[keep])


def test_ragged_grpo_workload():
    """32 responses (4 prompts x 8), lengths U{256..6912}, Bernoulli rewards,
    old/ref = new + N(0, 0.05^2) / N(0, 0.1^2), C=2, eps 0.2/0.28, beta=0.01."""
    w = synth.workload("grpo")
    lengths = synth.response_lengths(w)
    cu, lp_new, lp_old, lp_ref = _inputs(4, lengths)
    r = synth.rewards(w)
    A = OG.advantages(r, 8)
    o = OG.token_loss(lp_new, lp_old, lp_ref, cu, A)
    print(f"  rlk_grpo_token_loss T_tot={cu[-1]} B={len(lengths)}", flush=True)
    out = rlk.grpo_token_loss(f32_to_device(lp_new), f32_to_device(lp_old), f32_to_device(lp_ref),
                              cu, rewards=r, group_size=8)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(out["advantages"]), A, rtol=1e-6)
    _compare(out, o, o.near_branch)
    # larger noise exercises every branch (clip high/low, TIS cap)
    cu, lp_new, lp_old, lp_ref = _inputs(5, lengths, sd_old=0.6, sd_ref=0.5)
    o = OG.token_loss(lp_new, lp_old, lp_ref, cu, A)
    assert (o.flags & OG.FLAG_TIS).any() and (o.flags & OG.FLAG_CLIP).any()
    out = rlk.grpo_token_loss(f32_to_device(lp_new), f32_to_device(lp_old), f32_to_device(lp_ref),
                              cu, rewards=r, group_size=8)
    _compare(out, o, o.near_branch)


def test_advantages_mode_zero_length_and_params():
    lengths = [5, 0, 17, 1, 0, 300, 2, 9]
    cu, lp_new, lp_old, lp_ref = _inputs(6, lengths, sd_old=0.4, sd_ref=0.3)
    A = np.random.default_rng(7).normal(0, 1, len(lengths)).astype(np.float32)
    prm = OG.Params(tis_cap=1.5, eps_low=0.1, eps_high=0.2, kl_coef=0.05)
    o = OG.token_loss(lp_new, lp_old, lp_ref, cu, A.astype(np.float64), prm)
    out = rlk.grpo_token_loss(f32_to_device(lp_new), f32_to_device(lp_old), f32_to_device(lp_ref),
                              cu, advantages=A, tis_cap=1.5, eps_low=0.1, eps_high=0.2,
                              kl_coef=0.05)
    _compare(out, o, o.near_branch)


def test_on_policy_equal_lengths_is_zero_and_empty_batch():
    cu = synth.cu_seqlens(np.full(16, 40))
    lp = np.random.default_rng(8).normal(-1, 1, int(cu[-1])).astype(np.float32)
    r = np.array([1, 0, 0, 1, 1, 1, 0, 0] * 2, dtype=np.float32)
    x = f32_to_device(lp)
    out = rlk.grpo_token_loss(x, x, x, cu, rewards=r, group_size=8)
    assert abs(float(host(out["loss"]))) < 1e-7
    out = rlk.grpo_token_loss(x[:0], x[:0], x[:0], np.zeros(3, np.int64), rewards=r[:2],
                              group_size=2)
    assert float(host(out["loss"])) == 0.0


def test_bitwise_deterministic():
    w = synth.workload("grpo")
    cu, lp_new, lp_old, lp_ref = _inputs(9, synth.response_lengths(w))
    args = [f32_to_device(a) for a in (lp_new, lp_old, lp_ref)]
    r = synth.rewards(w)
    a = rlk.grpo_token_loss(*args, cu, rewards=r, group_size=8)
    b = rlk.grpo_token_loss(*args, cu, rewards=r, group_size=8)
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("loss_type,correction,aggregation,filt,baseline", [
    ("ipo", "tis", "token_mean", False, "mean"),
    ("icepop", "tis", "prompt_mean", True, "mean"),
    ("cispo", "mis", "token_mean", True, "length"),
    ("dapo", "mis", "prompt_mean", False, "length"),
    ("dapo", "tis", "prompt_mean", True, "length"),
    ("tis_pg", "tis", "token_mean", False, "mean"),
    ("tis_pg", "mis", "prompt_mean", True, "mean"),
])
def test_loss_variants(loss_type, correction, aggregation, filt, baseline):
    """The loss variants on the config-4 lengths with noisy ratios (every mask
    and clip branch taken), Bernoulli rewards (zero-advantage groups occur)."""
    w = synth.workload("grpo")
    lengths = synth.response_lengths(w)
    cu, lp_new, lp_old, lp_ref = _inputs(6, lengths, sd_old=0.6, sd_ref=0.5)
    r = synth.rewards(w)
    r[8:16] = 1.0                                  # one group with equal rewards: A = 0
    kw = dict(loss_type=loss_type, correction=correction, aggregation=aggregation,
              filter_zero_adv=filt, baseline=baseline, ipo_eps=0.1, icepop_lo=0.6,
              icepop_hi=1.5)
    prm = OG.Params(**kw)
    A = OG.advantages(r, 8, prm, lengths=lengths)
    assert np.any(A == 0.0)
    o = OG.token_loss(lp_new, lp_old, lp_ref, cu, A, prm, group_size=8)
    assert (o.flags & OG.FLAG_CLIP).any() or loss_type == "tis_pg"
    print(f"  rlk_grpo_token_loss T_tot={cu[-1]} {kw}", flush=True)
    out = rlk.grpo_token_loss(f32_to_device(lp_new), f32_to_device(lp_old), f32_to_device(lp_ref),
                              cu, rewards=r, group_size=8, **kw)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(out["advantages"]), A, rtol=1e-6, atol=1e-7)
    _compare(out, o, o.near_branch)
    if filt:                                       # filtered responses get no gradient
        Atok = np.repeat(A, np.diff(cu))
        assert not host(out["grad"])[Atok == 0.0].any()


def test_variants_with_advantages_given():
    """Advantages mode with prompt-mean aggregation (groups of 4) and IPO."""
    lengths = np.array([3, 0, 5, 2, 7, 1, 4, 4])
    cu, lp_new, lp_old, lp_ref = _inputs(7, lengths, sd_old=0.8)
    A = np.array([0.5, -0.5, 0.0, 1.0, 0.0, 0.0, 0.0, 0.0], dtype=np.float32)
    kw = dict(loss_type="ipo", aggregation="prompt_mean", filter_zero_adv=True, ipo_eps=0.05)
    prm = OG.Params(**kw)
    o = OG.token_loss(lp_new, lp_old, lp_ref, cu, A.astype(np.float64), prm, group_size=4)
    out = rlk.grpo_token_loss(f32_to_device(lp_new), f32_to_device(lp_old), f32_to_device(lp_ref),
                              cu, advantages=A, group_size=4, **kw)
    torch.cuda.synchronize()
    _compare(out, o, o.near_branch)


@pytest.mark.parametrize("kw", [dict(adv_eps=0.0), dict(adv_eps=0.0, baseline="length"),
                                dict(adv_eps=0.0, std_ddof=0), dict(normalize_std=False)])
def test_constant_reward_groups_give_zero_advantages(kw):
    """Groups whose rewards are all equal (all-correct / all-wrong, or any
    constant) get A = 0 exactly, with adv_eps = 0 too: no NaN reaches the loss,
    and zero-advantage filtering drops them."""
    lengths = np.arange(5, 37)
    cu, lp_new, lp_old, lp_ref = _inputs(11, lengths, sd_old=0.3)
    r = synth.rewards(synth.workload("grpo"))
    r[0:8], r[8:16], r[24:32] = 1.0, 0.0, 0.3
    prm = OG.Params(filter_zero_adv=True, **kw)
    A = OG.advantages(r, 8, prm, lengths=lengths)
    assert np.all(A[:16] == 0.0) and np.all(A[24:] == 0.0) and np.all(np.isfinite(A))
    o = OG.token_loss(lp_new, lp_old, lp_ref, cu, A, prm, group_size=8)
    print(f"  rlk_grpo_token_loss constant groups {kw}", flush=True)
    out = rlk.grpo_token_loss(f32_to_device(lp_new), f32_to_device(lp_old), f32_to_device(lp_ref),
                              cu, rewards=r, group_size=8, filter_zero_adv=True, **kw)
    torch.cuda.synchronize()
    adv = host(out["advantages"])
    assert np.all(adv[:16] == 0.0) and np.all(adv[24:] == 0.0)
    np.testing.assert_allclose(adv, A, rtol=1e-6, atol=1e-7)
    _compare(out, o, o.near_branch)
    assert int(host(out["status"])) == 0


def test_device_offsets_and_their_device_check():
    """cu_seqlens given as a device tensor is used in place; offsets that are
    not non-decreasing from 0 to the token count give NaN outputs and status 1
    (nothing is read on the host), and a valid call afterwards is unaffected."""
    lengths = np.array([4, 0, 9, 3, 6, 1, 2, 5])
    cu, lp_new, lp_old, lp_ref = _inputs(12, lengths, sd_old=0.3)
    args = [f32_to_device(a) for a in (lp_new, lp_old, lp_ref)]
    r = np.array([1, 0, 1, 1, 0, 0, 1, 0], dtype=np.float32)
    cu_dev = torch.from_numpy(cu).to("cuda:0")
    good = rlk.grpo_token_loss(*args, cu_dev, rewards=r, group_size=4)
    o = OG.token_loss(lp_new, lp_old, lp_ref, cu, OG.advantages(r, 4))
    torch.cuda.synchronize()
    _compare(good, o, o.near_branch)
    assert int(host(good["status"])) == 0
    T = int(cu[-1])
    for bad in ([1, 4, 4, 13, 16, 22, 23, 25, T], [0, 4, 3, 13, 16, 22, 23, 25, T],
                [0, 4, 4, 13, 16, 22, 23, 25, T - 1], [0, 4, 4, 13, 16, 22, 23, 25, T + 1]):
        cb = torch.tensor(bad, dtype=torch.int64, device="cuda:0")
        print(f"  rlk_grpo_token_loss invalid offsets {bad}", flush=True)
        out = rlk.grpo_token_loss(*args, cb, rewards=r, group_size=4)
        torch.cuda.synchronize()
        assert int(host(out["status"])) == 1
        assert np.isnan(float(host(out["loss"])))
        assert np.isnan(host(out["grad"])).all() and np.isnan(host(out["token_loss"])).all()
        assert np.isnan(host(out["metrics"])).all() and np.isnan(host(out["advantages"])).all()
        assert not host(out["token_flags"]).any()
    again = rlk.grpo_token_loss(*args, cu_dev, rewards=r, group_size=4)
    for k in good:
        assert torch.equal(good[k], again[k]), k


def test_many_tokens():
    """About 10^7 packed tokens (32 responses of 2^17..2^19 tokens): tens of
    thousands of 256-token partials folded in one fixed order."""
    rng = np.random.default_rng(31)
    lengths = rng.integers(1 << 17, 1 << 19, 32)
    cu, lp_new, lp_old, lp_ref = _inputs(8, lengths, sd_old=0.3, sd_ref=0.2)
    r = rng.integers(0, 2, 32).astype(np.float32)
    A = OG.advantages(r, 8)
    print(f"  oracle loss T_tot={cu[-1]}", flush=True)
    o = OG.token_loss(lp_new, lp_old, lp_ref, cu, A)
    print(f"  rlk_grpo_token_loss T_tot={cu[-1]} B={len(lengths)}", flush=True)
    out = rlk.grpo_token_loss(f32_to_device(lp_new), f32_to_device(lp_old), f32_to_device(lp_ref),
                              cu, rewards=r, group_size=8)
    torch.cuda.synchronize()
    _compare(out, o, o.near_branch)
