"""fp64 oracle: seeded Gumbel-max draw of a target token from the nucleus.

TEST INFRASTRUCTURE ONLY (see the package docstring). ``gumbel_max_target``
prepares test inputs from given uniforms; ``sample_row`` is the definition the
GPU sampler (rlk_sample_top_p) is checked against.

The rollout side samples from the same truncated distribution the trainer
scores (prime-rl v0.10.0 release notes, "2. RL Algorithms": top-p sampling is
replayed exactly in the trainer). Gumbel-max: with u_i uniform on (0, 1),
y = argmax_{i in S} (d_i + g_i), g_i = -log(-log u_i), the lowest index on an
exact tie. This draws y with probability exp(d_y) / Z_S.
"""
from __future__ import annotations

import numpy as np

from . import logprob, philox


def gumbel_max_target(z, T: float, p: float, u, top_k: int = 0) -> int:
    """Target id drawn from the top-k/top-p nucleus of row ``z`` with uniforms ``u``."""
    z = np.asarray(z, dtype=np.float64)
    keep, *_ = logprob.nucleus(z, T, p, top_k)
    m = z[keep].max()
    score = np.full(z.size, -np.inf)
    score[keep] = (z[keep] - m) / T - np.log(-np.log(np.asarray(u, dtype=np.float64)[keep]))
    return int(np.argmax(score))


def sample_row(z, T: float, p: float, seed: int, offset: int, row_key: int,
               top_k: int = 0) -> int:
    """The GPU sampler's definition: Gumbel-max over the top-k/top-p nucleus
    of the tempered row with Philox uniforms (``philox.row_uniforms``):
    y = argmax_{i in S} (z_i / T - log(-log u_i)), the lowest id on an exact
    tie; -1 for a row with a NaN / +inf logit or no finite logit. The score
    drops the row max the other form subtracts: the same argmax and law."""
    z = np.asarray(z, dtype=np.float64)
    if np.isnan(z).any() or np.isposinf(z).any() or not (z > -np.inf).any():
        return -1
    keep, *_ = logprob.nucleus(z, T, p, top_k)
    u = philox.row_uniforms(seed, offset, row_key, z.size)
    score = np.full(z.size, -np.inf)
    score[keep] = z[keep] / T - np.log(-np.log(u[keep]))
    return int(np.argmax(score))
