"""fp64 oracle: the fused LM-head forms (forward and backward).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Forward. logits z = h . W^T, formed in fp64 from the bf16-exact operands and
never rounded (the kernel accumulates in fp32 and keeps the logits unrounded),
then the row statistics of ``oracle.logprob`` at the given T and p. The
entropy output of the fused form is the truncated one, which is the full one
at p = 1. The pages' "chunked torchtitan-style" loss (prime-rl v0.10.0
release notes, "1. Trainer Performance") is the same quantity computed
without holding all logits at once; the oracle simply materialises them.

Backward. For a scalar loss L with per-row upstream gradients
g_lp = dL/dlp and g_H = dL/dH (already divided by the token count: the loss
seed is normalised before model derivatives, Qwen3-8B VIME consistency page,
"Canonical topology strategy"), with q_i = exp(d_i) / Z_S on the nucleus S
(S held fixed, i.e. the cut is treated as a constant):

  dL/dz_{n,i} = (1/T) [ g_lp (delta_{i,y} - q_i) - g_H q_i (d_i - sum_{j in S} q_j d_j) ]
                for i in S, and 0 outside S;
  dL/dh = G . W,     dL/dW = G^T . h,     G = [dL/dz].

This follows from dlp/dd_i = delta_{iy} - q_i and dH/dd_i = -q_i (d_i - E_q d)
on S, with dd_i/dz_i = 1/T. A row whose target is outside S has lp = -inf;
its lp term is dropped (only the entropy term contributes).
"""
from __future__ import annotations

import numpy as np

from . import logprob


def logits(h64: np.ndarray, w64: np.ndarray) -> np.ndarray:
    """fp64 logits [N, V] from fp64 hidden [N, H] and weight [V, H]."""
    return np.asarray(h64, dtype=np.float64) @ np.asarray(w64, dtype=np.float64).T


def forward(h64, w64, targets, T: float, p: float, top_k: int = 0) -> logprob.BatchResult:
    """Per-row outputs of the fused form (truncated statistics; full at p = 1
    without top-k)."""
    return logprob.logprob_from_logits(logits(h64, w64), targets, T, p, top_k)


def grad_logits(z: np.ndarray, targets, g_lp, g_H, T: float, p: float,
                top_k: int = 0) -> np.ndarray:
    """G = dL/dz [N, V] for per-row upstream gradients g_lp, g_H (S the
    top-k/top-p nucleus, held fixed)."""
    z = np.asarray(z, dtype=np.float64)
    N, V = z.shape
    G = np.zeros((N, V))
    for n in range(N):
        keep, *_ = logprob.nucleus(z[n], T, p, top_k)
        zk = z[n, keep]
        d = (zk - zk.max()) / T
        e = np.exp(d)
        q = e / e.sum()
        Ed = (q * d).sum()
        y = int(targets[n])
        onehot = np.zeros(V)
        lp_term = 0.0 <= y < V and keep[y]
        if lp_term:
            onehot[y] = 1.0
        g = -float(g_H[n]) * q * (d - Ed)
        if lp_term:
            g = g + float(g_lp[n]) * (onehot[keep] - q)
        G[n, keep] = g / T
    return G


def backward(h64, w64, targets, g_lp, g_H, T: float, p: float, top_k: int = 0):
    """(dL/dh [N, H], dL/dW [V, H]) in fp64."""
    h64 = np.asarray(h64, dtype=np.float64)
    w64 = np.asarray(w64, dtype=np.float64)
    G = grad_logits(logits(h64, w64), targets, g_lp, g_H, T, p, top_k)
    return G @ w64, G.T @ h64
