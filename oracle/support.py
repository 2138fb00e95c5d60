"""fp64 oracle: log-probability and entropy over a caller-supplied retained set.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages: Qwen3-8B VIME train-rollout consistency page, "ROCm MI300X and
gfx942": below top-p 1 the rollout sampler hands its complete finite
retained-token set to the deterministic logprob kernel, and the sparse HIP
path scores the selected token and the monitoring entropy over that set;
prime-rl v0.10.0 release notes, "Breaking changes": the sampling mask
travels in CSR form. The pages give no formula; the plain reading is the
distribution renormalised over the supplied set, with temperature first:

For row n with support S = ids[offsets[n] : offsets[n + 1]]:
  m     = max_{i in S} z_i
  d_i   = (z_i - m) / T
  Z_S   = sum_{i in S} exp(d_i)
  lp    = d_y - log Z_S            if y in S, else -inf (flag bit 0)
  H     = log Z_S - sum_{i in S} exp(d_i) d_i / Z_S

A valid support is non-empty, in range and strictly increasing (the CSR form
of a boolean mask), and its logits are finite (the pages' set is finite).
Flags (uint8): bit0 target not in S; bit1 target out of range (lp NaN);
bit2 a non-finite logit in S (outputs NaN); bit5 invalid support (outputs
NaN). With a top-p value to check against: bit6 when S is none of the valid
nuclei of the row at (T, p) (``logprob.nucleus``: the nucleus, or on a
boundary row one of its alternatives), bit3 when the row is such a boundary
row.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import logprob

FLAG_OUTSIDE = logprob.FLAG_OUTSIDE
FLAG_BAD_TARGET = logprob.FLAG_BAD_TARGET
FLAG_NONFINITE = logprob.FLAG_NONFINITE
FLAG_BOUNDARY = logprob.FLAG_BOUNDARY
FLAG_BAD_SUPPORT = 32
FLAG_MISMATCH = 64


def valid_support(ids, V: int) -> bool:
    """Non-empty, every id in [0, V), strictly increasing."""
    ids = np.asarray(ids, dtype=np.int64)
    return ids.size > 0 and bool(np.all((ids >= 0) & (ids < V))) and bool(np.all(np.diff(ids) > 0))


def row(z, y: int, T: float, ids, check_p: float | None = None,
        check_k: int = 0) -> tuple[float, float, int]:
    """(lp, H, flags) of one row over the support ``ids``; with ``check_p``
    the set is compared with the row's top-k/top-p nucleus (k = ``check_k``)."""
    z = np.asarray(z, dtype=np.float64)
    V = z.size
    ids = np.asarray(ids, dtype=np.int64)
    flags = 0
    bad_target = not (0 <= y < V)
    if bad_target:
        flags |= FLAG_BAD_TARGET
    nan = float("nan")
    if not valid_support(ids, V):
        return nan, nan, flags | FLAG_BAD_SUPPORT
    zs = z[ids]
    if not np.all(np.isfinite(zs)):
        return nan, nan, flags | FLAG_NONFINITE
    m = zs.max()
    d = (zs - m) / T
    e = np.exp(d)
    Zs = e.sum()
    logZs = np.log(Zs)
    h = float(logZs - (e * d).sum() / Zs)
    if bad_target:
        lp = nan
    else:
        hit = np.flatnonzero(ids == y)
        if hit.size:
            lp = float(d[hit[0]] - logZs)
        else:
            lp = -np.inf
            flags |= FLAG_OUTSIDE
    if check_p is not None and not (np.isnan(z).any() or np.isposinf(z).any()):
        keep, _, _, _, alts = logprob.nucleus(z, T, check_p, check_k)
        mask = np.zeros(V, dtype=bool)
        mask[ids] = True
        if alts:
            flags |= FLAG_BOUNDARY
        if not any(np.array_equal(mask, k) for k in [keep] + alts):
            flags |= FLAG_MISMATCH
    return lp, h, flags


@dataclasses.dataclass
class SupportResult:
    lp: np.ndarray
    h: np.ndarray
    size: np.ndarray
    flags: np.ndarray


def logprob_from_support(logits, targets, T: float, offsets, ids,
                         check_p: float | None = None, check_k: int = 0) -> SupportResult:
    """Row-wise outputs for [N, V] logits and a CSR support (offsets [N + 1], ids)."""
    logits = np.asarray(logits, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    N = logits.shape[0]
    out = SupportResult(np.empty(N), np.empty(N), np.empty(N, dtype=np.int64),
                        np.empty(N, dtype=np.uint8))
    for n in range(N):
        s = ids[offsets[n]:offsets[n + 1]]
        out.lp[n], out.h[n], out.flags[n] = row(logits[n], int(targets[n]), T, s, check_p, check_k)
        out.size[n] = offsets[n + 1] - offsets[n]
    return out


def csr_from_masks(masks) -> tuple[np.ndarray, np.ndarray]:
    """CSR (offsets int64 [N + 1], ids int32) of boolean row masks."""
    masks = np.asarray(masks, dtype=bool)
    counts = masks.sum(axis=1)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    ids = np.concatenate([np.flatnonzero(m) for m in masks]).astype(np.int32) \
        if masks.shape[0] else np.zeros(0, dtype=np.int32)
    return offsets, ids
