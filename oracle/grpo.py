"""fp64 oracle: group-normalised advantages and the GRPO/DAPO token loss.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name GRPO and DAPO (LumenRL README, "Key Features"), GRPO standard-
deviation normalisation and eight samples per prompt (RL-Kernel ROCm sparse
performance page, profile paragraph), a KL coefficient of 0.01 (same page,
quick-start command), and truncated importance sampling that "clips large
ratios" (LumenRL README, "Rollout Correction"). They give no formulas. The
plain reading used here, for response j in group g (consecutive blocks of
``group_size`` responses) and token t of response j:

  advantages   A_j  = (r_j - mean_g r) / (std_g r + adv_eps)   (std with ``ddof``;
                      without std normalisation A_j = r_j - mean_g r);
                      A_j = 0 for every response of a group whose rewards
                      are all equal (a constant group gives A = 0)
  ratio        rho_t = exp(lp_new_t - lp_old_t)
  TIS          rho~_t = min(rho_t, C)
  surrogate    s_t  = min(rho~_t A_j, clip(rho~_t, 1 - eps_low, 1 + eps_high) A_j)
  k3 KL        delta_t = lp_ref_t - lp_new_t,  k3_t = exp(delta_t) - delta_t - 1
  token loss   l_t  = -s_t + beta k3_t
  loss         L    = sum_t l_t / T_tot   (token mean over every response token)

Gradient with respect to lp_new (lp_old, lp_ref and A are constants):

  dL/dlp_new_t = ( -A_j rho_t active_t + beta (1 - exp(delta_t)) ) / T_tot
  active_t = (rho_t <= C) and not (A_j > 0 and rho_t > 1 + eps_high)
                          and not (A_j < 0 and rho_t < 1 - eps_low)

At an exact equality point (rho = C, rho = 1 + eps_high, rho = 1 - eps_low)
the untruncated, unclipped derivative is used.

Token flags: bit0 the TIS cap binds (rho > C); bit1 the clipped branch is the
one taken by the min (A > 0 and rho~ > 1 + eps_high, or A < 0 and
rho~ < 1 - eps_low). Metrics (token means): clip fraction (bit1), TIS fraction
(bit0), k3, rho.

Variants (prime-rl v0.10.0 release notes, "2. RL Algorithms": IPO masks a
token when |pi_train - pi_infer| > eps, eps = 0.3, no KL term; IcePop masks
it when pi_train / pi_infer leaves a fixed band; CISPO and PPO stay opt-in;
GRPO gains a length-weighted baseline and exact prompt-mean aggregation;
"Breaking changes": zero-advantage samples are filtered. LumenRL README,
"Rollout Correction": MIS normalises the ratios). pi_infer is exp(lp_old)
(the rollout's logprob), pi_train is exp(lp_new). Plain readings:

  correction   tis: rho~ = min(rho, C);  mis: rho~ = rho / mean(rho) over the
               tokens that enter the loss, the mean held constant
  dapo         as above
  ipo          m = [|exp(lp_new) - exp(lp_old)| <= eps_ipo];  s = m rho~ A
  icepop       m = [band_lo <= rho <= band_hi];              s = m rho~ A
  cispo        w = clip(rho~, 1 - eps_low, 1 + eps_high) held constant;
               s = w A lp_new (its gradient is w A)
  tis_pg       the detached-TIS form: rho~ a constant weight on an on-policy
               surrogate whose proximal policy is lp_new itself, so the
               surrogate's ratio is 1 at the evaluation point: s = rho~ A,
               gradient rho~ A (no clip can bind)
  baseline     mean: mean_g r;  length: sum_j L_j r_j / sum_j L_j (L_j tokens)
  filter       a response with A_j == 0 is left out of the loss and its count
  aggregation  token_mean: every kept token weighs 1 / T_kept;
               prompt_mean: a kept token of group g weighs 1 / (G_kept T_g),
               T_g the kept tokens of group g, G_kept the groups with T_g > 0

The ratio part of the gradient is -A rho~ times the indicator that the
chosen branch depends on lp_new (TIS: rho <= C; dapo: the unclipped branch;
ipo/icepop: m; cispo: always, with w in place of rho~). Flags bit1 marks the
clipped branch (dapo), a masked token (ipo, icepop) or a binding clip on w
(cispo).
"""
from __future__ import annotations

import dataclasses

import numpy as np

FLAG_TIS = 1
FLAG_CLIP = 2


@dataclasses.dataclass
class Params:
    tis_cap: float = 2.0
    eps_low: float = 0.2
    eps_high: float = 0.28
    kl_coef: float = 0.01
    adv_eps: float = 1e-6
    std_ddof: int = 1
    normalize_std: bool = True
    loss_type: str = "dapo"        # dapo | ipo | icepop | cispo | tis_pg
    correction: str = "tis"        # tis | mis
    aggregation: str = "token_mean"   # token_mean | prompt_mean
    filter_zero_adv: bool = False
    baseline: str = "mean"         # mean | length
    ipo_eps: float = 0.3
    icepop_lo: float = 0.5
    icepop_hi: float = 2.0


def advantages(rewards, group_size: int, prm: Params = Params(), lengths=None) -> np.ndarray:
    """Per-response advantages, groups of ``group_size`` consecutive responses
    (``lengths``: response token counts, for the length-weighted baseline)."""
    r = np.asarray(rewards, dtype=np.float64).reshape(-1, group_size)
    if prm.baseline == "length":
        L = np.asarray(lengths, dtype=np.float64).reshape(-1, group_size)
        tot = L.sum(axis=1, keepdims=True)
        b = np.where(tot > 0, (L * r).sum(axis=1, keepdims=True) / np.where(tot > 0, tot, 1.0),
                     r.mean(axis=1, keepdims=True))
    else:
        b = r.mean(axis=1, keepdims=True)
    mu = r.mean(axis=1, keepdims=True)
    a = r - b
    if prm.normalize_std:
        sd = np.sqrt(((r - mu) ** 2).sum(axis=1, keepdims=True) / (group_size - prm.std_ddof))
        with np.errstate(invalid="ignore", divide="ignore"):
            a = a / (sd + prm.adv_eps)
    # a group whose rewards are all equal carries no signal: its advantages are
    # exactly 0 (its std and every r_j - baseline vanish), also with adv_eps = 0
    # where the quotient above would be 0/0
    const = (r == r[:, :1]).all(axis=1, keepdims=True)
    a = np.where(const, 0.0, a)
    return a.reshape(-1)


@dataclasses.dataclass
class LossResult:
    loss: float
    grad: np.ndarray         # dL/dlp_new [T_tot]
    token_loss: np.ndarray   # l_t [T_tot]
    flags: np.ndarray        # uint8 [T_tot]
    metrics: np.ndarray      # [clip frac, TIS frac, mean k3, mean rho]
    near_branch: np.ndarray  # bool [T_tot]: rho within rel 1e-6 of a branch point


def weights(cu_seqlens, adv, group_size: int, prm: Params = Params()) -> np.ndarray:
    """Per-token loss weights of the aggregation (0 for a filtered response)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    L = np.diff(cu).astype(np.float64)
    A = np.asarray(adv, dtype=np.float64)
    keep = ~(prm.filter_zero_adv & (A == 0.0)) if prm.filter_zero_adv else np.ones(A.size, bool)
    if prm.aggregation == "prompt_mean":
        Tg = (L * keep).reshape(-1, group_size).sum(axis=1)
        G_kept = int((Tg > 0).sum())
        wj = np.where(keep, 1.0 / np.maximum(G_kept * np.repeat(Tg, group_size), 1e-300), 0.0)
        if G_kept == 0:
            wj[:] = 0.0
    else:
        T_kept = float((L * keep).sum())
        wj = np.where(keep, 1.0 / T_kept if T_kept > 0 else 0.0, 0.0)
    return np.repeat(wj, np.diff(cu))


def token_loss(lp_new, lp_old, lp_ref, cu_seqlens, adv, prm: Params = Params(),
               group_size: int = 1) -> LossResult:
    """The aggregated loss, its gradient, per-token terms and metrics."""
    lp_new = np.asarray(lp_new, dtype=np.float64)
    lp_old = np.asarray(lp_old, dtype=np.float64)
    lp_ref = np.asarray(lp_ref, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T_tot = int(cu[-1])
    A = np.repeat(np.asarray(adv, dtype=np.float64), np.diff(cu))
    C, lo, hi, beta = prm.tis_cap, 1.0 - prm.eps_low, 1.0 + prm.eps_high, prm.kl_coef
    if T_tot == 0:
        return LossResult(0.0, np.zeros(0), np.zeros(0), np.zeros(0, np.uint8), np.zeros(4),
                          np.zeros(0, bool))
    wt = weights(cu, adv, group_size, prm)
    rho = np.exp(lp_new - lp_old)
    if prm.correction == "mis":
        used = wt > 0
        rbar = rho[used].mean() if used.any() else 1.0
        rt = rho / rbar
        tis = np.zeros(T_tot, bool)
        ratio_live = np.ones(T_tot, bool)
    else:
        rt = np.minimum(rho, C)
        tis = rho > C
        ratio_live = rho <= C
    delta = lp_ref - lp_new
    k3 = np.exp(delta) - delta - 1.0
    if prm.loss_type == "dapo":
        s = np.minimum(rt * A, np.clip(rt, lo, hi) * A)
        flag2 = ((A > 0) & (rt > hi)) | ((A < 0) & (rt < lo))
        live = ratio_live & ~flag2
        g_ratio = -A * rt * live
    elif prm.loss_type in ("ipo", "icepop"):
        if prm.loss_type == "ipo":
            m = np.abs(np.exp(lp_new) - np.exp(lp_old)) <= prm.ipo_eps
        else:
            m = (rho >= prm.icepop_lo) & (rho <= prm.icepop_hi)
        s = m * rt * A
        flag2 = ~m
        g_ratio = -A * rt * (m & ratio_live)
    elif prm.loss_type == "tis_pg":
        s = rt * A
        flag2 = np.zeros(T_tot, bool)
        g_ratio = -A * rt
    elif prm.loss_type == "cispo":
        w = np.clip(rt, lo, hi)
        s = w * A * lp_new
        flag2 = (rt < lo) | (rt > hi)
        g_ratio = -A * w
    else:
        raise ValueError(prm.loss_type)
    ell = -s + beta * k3
    flags = (tis * FLAG_TIS + flag2 * FLAG_CLIP).astype(np.uint8)
    grad = wt * (g_ratio + beta * (1.0 - np.exp(delta)))
    metrics = np.array([flag2.mean(), tis.mean(), k3.mean(), rho.mean()])
    near = np.zeros(T_tot, dtype=bool)
    bps = [lo, hi] + ([C] if prm.correction == "tis" else [])
    if prm.loss_type == "icepop":
        bps += [prm.icepop_lo, prm.icepop_hi]
    for b in bps:
        near |= np.abs(rt - b) <= 1e-6 * b
        near |= np.abs(rho - b) <= 1e-6 * b
    if prm.loss_type == "ipo":
        near |= np.abs(np.abs(np.exp(lp_new) - np.exp(lp_old)) - prm.ipo_eps) <= 1e-6
    return LossResult(float((wt * ell).sum()), grad, ell, flags, metrics, near)
