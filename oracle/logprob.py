"""fp64 oracle: tempered full-vocabulary and top-p truncated log-probability / entropy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definitions (pages: Qwen3-8B VIME train-rollout consistency, section "ROCm
MI300X and gfx942": temperature finite and positive, top-p in (0, 1], the
complete retained-token set is scored, top-p = 1 means the full vocabulary;
RL-Kernel ROCm sparse performance page, quick-start command: temperature 0.7,
top-p 0.95; the same section names the entropy as "monitoring entropy").
The pages give names, not formulas; the readings below are the plain ones.

For one row of logits z[0..V) and target y:

  m      = max_i z_i over finite entries
  d_i    = (z_i - m) / T                    (temperature before top-p)
  Z      = sum_i exp(d_i)
  lp     = d_y - log Z
  H      = log Z - sum_i exp(d_i) d_i / Z   (nats)

Nucleus S (top-p, keep-all-ties reading):
  tokens are ordered by z descending; equal values form one group.
  M_>(v) = mass strictly above v, M_>=(v) = mass at or above v.
  p = 1: S = all finite tokens.
  p < 1: tau = the lowest row value v with M_>(v) < p;  S = {z >= tau}.
  Equivalently: walk groups from the top, stop at the first group whose
  inclusive cumulative mass reaches p, keep that whole group.

Top-k (opt-in, k > 0; the consistency page's strict contract rejects it, the
prime-rl release notes replay it in the trainer): first S_k = {z >= v_k}
with v_k the k-th largest finite value (ties with it kept, so |S_k| >= k; k
at or above the number of finite values keeps them all), then the top-p rule
above on the distribution renormalised over S_k (masses relative to
Z_k = sum_{i in S_k} exp(d_i)); p = 1 keeps S_k and reports tau = v_k.

Truncated, renormalised distribution over S:
  Z_S      = sum_{i in S} exp(d_i)
  lp_trunc = d_y - log Z_S   if y in S, else -inf (flag bit 0)
  H_trunc  = log Z_S - sum_{i in S} exp(d_i) d_i / Z_S

Per-row flags (uint8): bit0 target outside the nucleus, bit1 target out of
range (outputs NaN), bit2 a NaN/+inf logit or no finite logit (outputs NaN),
bit3 the row lies within BOUNDARY_EPS of the p boundary (either M_>(tau) or
M_>=(tau) is within 1e-6 of p), where another equally valid set exists.
"""
from __future__ import annotations

import dataclasses

import numpy as np

FLAG_OUTSIDE = 1
FLAG_BAD_TARGET = 2
FLAG_NONFINITE = 4
FLAG_BOUNDARY = 8

BOUNDARY_EPS = 1e-6


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f32(x: float) -> float:
    """The fp32 value a scalar parameter takes when passed through the C ABI."""
    return float(np.float32(x))


@dataclasses.dataclass
class RowResult:
    lp_full: float
    h_full: float
    lp_trunc: float
    h_trunc: float
    size: int            # |S|
    tau: float           # cut value (-inf when p == 1)
    m_gt: float          # M_>(tau)
    m_ge: float          # M_>=(tau)
    flags: int
    keep: np.ndarray     # bool mask of S
    alt_keeps: list      # other valid nucleus masks for a boundary row


def _nan_row(V: int, flags: int) -> RowResult:
    nan = float("nan")
    return RowResult(nan, nan, nan, nan, 0, nan, nan, nan, flags,
                     np.zeros(V, dtype=bool), [])


def top_k_floor(z, top_k: int) -> float:
    """v_k, the k-th largest finite value of the row (ties counted one by
    one), or -inf when top-k is off (k = 0) or keeps every finite value."""
    z = np.asarray(z, dtype=np.float64)
    fin = np.sort(z[z > -np.inf])[::-1]
    if top_k <= 0 or top_k >= fin.size:
        return -np.inf
    return float(fin[top_k - 1])


def nucleus(z, T: float, p: float, top_k: int = 0):
    """Top-k then top-p nucleus of one row by sorting (the plain definition).

    Returns (keep mask, tau, M_>(tau), M_>=(tau), alt masks). Masses are
    probabilities of the tempered distribution renormalised over the top-k
    set (the whole row without top-k). ``z`` must hold no NaN/+inf and at
    least one finite value.
    """
    z = np.asarray(z, dtype=np.float64)
    finite = z > -np.inf
    vk = top_k_floor(z, top_k)
    if vk > -np.inf:
        finite = z >= vk                  # S_k: the top-k set, ties with v_k kept
    if p >= 1.0:
        return finite.copy(), vk, 0.0, 1.0, []
    m = z[finite].max()
    e = np.where(finite, np.exp((z - m) / T), 0.0)
    order = np.argsort(-z, kind="stable")
    order = order[finite[order]]          # the candidates, largest first
    zs = z[order]
    c = np.cumsum(e[order])
    Z = c[-1]
    # last index of every group of equal values
    ends = np.flatnonzero(np.append(zs[1:] != zs[:-1], True))
    cg = c[ends] / Z
    g = int(np.argmax(cg >= p))          # first group whose inclusive mass reaches p
    tau = zs[ends[g]]
    m_gt = cg[g - 1] if g > 0 else 0.0
    m_ge = cg[g]
    keep = z >= tau
    alts = []
    if abs(m_gt - p) <= BOUNDARY_EPS and g > 0:
        alts.append(z > tau)             # the boundary group could fall out
    if abs(m_ge - p) <= BOUNDARY_EPS and g + 1 < ends.size:
        nxt = zs[ends[g + 1]]
        if nxt > -np.inf:
            alts.append(z >= nxt)        # the next group could come in
    return keep, float(tau), float(m_gt), float(m_ge), alts


def truncated(z, y: int, T: float, keep: np.ndarray) -> tuple[float, float]:
    """(lp_trunc, H_trunc) of the distribution renormalised over ``keep``."""
    z = np.asarray(z, dtype=np.float64)
    m = z[keep].max()
    d = (z[keep] - m) / T
    e = np.exp(d)
    Zs = e.sum()
    logZs = np.log(Zs)
    h_trunc = logZs - (e * d).sum() / Zs
    if not (0 <= y < z.size):
        return float("nan"), float(h_trunc)
    if not keep[y]:
        return -np.inf, float(h_trunc)
    return float((z[y] - m) / T - logZs), float(h_trunc)


def row(z, y: int, T: float, p: float, top_k: int = 0) -> RowResult:
    """All outputs for one row (fp64); ``top_k`` = 0: no top-k."""
    z = np.asarray(z, dtype=np.float64)
    V = z.size
    flags = 0
    bad_target = not (0 <= y < V)
    if bad_target:
        flags |= FLAG_BAD_TARGET
    if np.isnan(z).any() or np.isposinf(z).any() or not (z > -np.inf).any():
        return _nan_row(V, flags | FLAG_NONFINITE)
    finite = z > -np.inf
    m = z[finite].max()
    d = np.where(finite, (z - m) / T, -np.inf)
    e = np.exp(d)
    ed = np.where(finite, e * np.where(finite, d, 0.0), 0.0)
    Z = e.sum()
    logZ = np.log(Z)
    h_full = logZ - ed.sum() / Z
    keep, tau, m_gt, m_ge, alts = nucleus(z, T, p, top_k)
    if alts:
        flags |= FLAG_BOUNDARY
    lp_trunc, h_trunc = truncated(z, y, T, keep)
    if bad_target:
        lp_full = float("nan")
    else:
        lp_full = d[y] - logZ
        if not keep[y]:
            flags |= FLAG_OUTSIDE
    return RowResult(float(lp_full), float(h_full), float(lp_trunc), float(h_trunc),
                     int(keep.sum()), tau, m_gt, m_ge, flags, keep, alts)


@dataclasses.dataclass
class BatchResult:
    lp_full: np.ndarray
    h_full: np.ndarray
    lp_trunc: np.ndarray
    h_trunc: np.ndarray
    size: np.ndarray
    tau: np.ndarray
    flags: np.ndarray
    alts: list           # per row: [(|S'|, lp_trunc', H_trunc') for each other valid nucleus]


def logprob_from_logits(logits, targets, T, p, top_k=0) -> BatchResult:
    """Row-wise outputs for a [N, V] array of fp64-widened logits.

    ``T`` and ``p`` are scalars or per-row arrays (already the fp32 values the
    ABI receives, widened); ``top_k`` a scalar or per-row array (0: off).
    """
    logits = np.asarray(logits, dtype=np.float64)
    N = logits.shape[0]
    Ts = np.broadcast_to(np.asarray(T, dtype=np.float64), (N,))
    ps = np.broadcast_to(np.asarray(p, dtype=np.float64), (N,))
    ks = np.broadcast_to(np.asarray(top_k, dtype=np.int64), (N,))
    out = BatchResult(*(np.empty(N) for _ in range(4)), np.empty(N, dtype=np.int64),
                      np.empty(N), np.empty(N, dtype=np.uint8), [])
    for n in range(N):
        r = row(logits[n], int(targets[n]), float(Ts[n]), float(ps[n]), int(ks[n]))
        out.lp_full[n], out.h_full[n] = r.lp_full, r.h_full
        out.lp_trunc[n], out.h_trunc[n] = r.lp_trunc, r.h_trunc
        out.size[n], out.tau[n], out.flags[n] = r.size, r.tau, r.flags
        out.alts.append([(int(a.sum()),) + truncated(logits[n], int(targets[n]), float(Ts[n]), a)
                         for a in r.alt_keeps])
    return out
