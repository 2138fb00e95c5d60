"""fp64 oracle: seeded Gumbel-max draw of a target token from the nucleus.

TEST INFRASTRUCTURE ONLY (see the package docstring). It prepares inputs: the
HIP path never samples, it scores the target it is given.

The rollout side samples from the same truncated distribution the trainer
scores (prime-rl v0.10.0 release notes, "2. RL Algorithms": top-p sampling is
replayed exactly in the trainer). Gumbel-max: with u_i uniform on (0, 1),
y = argmax_{i in S} (d_i + g_i), g_i = -log(-log u_i), the lowest index on an
exact tie. This draws y with probability exp(d_y) / Z_S.
"""
from __future__ import annotations

import numpy as np

from . import logprob


def gumbel_max_target(z, T: float, p: float, u) -> int:
    """Target id drawn from the top-p nucleus of row ``z`` with uniforms ``u``."""
    z = np.asarray(z, dtype=np.float64)
    keep, *_ = logprob.nucleus(z, T, p)
    m = z[keep].max()
    score = np.full(z.size, -np.inf)
    score[keep] = (z[keep] - m) / T - np.log(-np.log(np.asarray(u, dtype=np.float64)[keep]))
    return int(np.argmax(score))
