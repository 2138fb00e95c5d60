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
                      without std normalisation A_j = r_j - mean_g r)
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


def advantages(rewards, group_size: int, prm: Params = Params()) -> np.ndarray:
    """Per-response advantages, groups of ``group_size`` consecutive responses."""
    r = np.asarray(rewards, dtype=np.float64).reshape(-1, group_size)
    mu = r.mean(axis=1, keepdims=True)
    a = r - mu
    if prm.normalize_std:
        sd = np.sqrt(((r - mu) ** 2).sum(axis=1, keepdims=True) / (group_size - prm.std_ddof))
        a = a / (sd + prm.adv_eps)
    return a.reshape(-1)


@dataclasses.dataclass
class LossResult:
    loss: float
    grad: np.ndarray         # dL/dlp_new [T_tot]
    token_loss: np.ndarray   # l_t [T_tot]
    flags: np.ndarray        # uint8 [T_tot]
    metrics: np.ndarray      # [clip frac, TIS frac, mean k3, mean rho]
    near_branch: np.ndarray  # bool [T_tot]: rho within rel 1e-6 of a branch point


def token_loss(lp_new, lp_old, lp_ref, cu_seqlens, adv, prm: Params = Params()) -> LossResult:
    """The ragged token-mean loss, its gradient, per-token terms and metrics."""
    lp_new = np.asarray(lp_new, dtype=np.float64)
    lp_old = np.asarray(lp_old, dtype=np.float64)
    lp_ref = np.asarray(lp_ref, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T_tot = int(cu[-1])
    A = np.repeat(np.asarray(adv, dtype=np.float64), np.diff(cu))
    C, lo, hi, beta = prm.tis_cap, 1.0 - prm.eps_low, 1.0 + prm.eps_high, prm.kl_coef
    rho = np.exp(lp_new - lp_old)
    rho_t = np.minimum(rho, C)
    s = np.minimum(rho_t * A, np.clip(rho_t, lo, hi) * A)
    delta = lp_ref - lp_new
    k3 = np.exp(delta) - delta - 1.0
    ell = -s + beta * k3
    active = (rho <= C) & ~((A > 0) & (rho > hi)) & ~((A < 0) & (rho < lo))
    tis = rho > C
    clip = ((A > 0) & (rho_t > hi)) | ((A < 0) & (rho_t < lo))
    flags = (tis * FLAG_TIS + clip * FLAG_CLIP).astype(np.uint8)
    if T_tot == 0:
        return LossResult(0.0, np.zeros(0), np.zeros(0), flags, np.zeros(4), np.zeros(0, bool))
    grad = (-A * rho * active + beta * (1.0 - np.exp(delta))) / T_tot
    metrics = np.array([clip.mean(), tis.mean(), k3.mean(), rho.mean()])
    near = np.zeros(T_tot, dtype=bool)
    for b in (C, lo, hi):
        near |= np.abs(rho - b) <= 1e-6 * b
    return LossResult(float(ell.sum() / T_tot), grad, ell, flags, metrics, near)
