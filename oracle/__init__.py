"""CPU fp64 oracle for token log-probabilities, entropy and the GRPO token loss.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its
Python binding) may import, call or link anything in this package; only the
tests, the smoke check and the benchmark's CPU-baseline leg use it.

It is a plain, slow, obviously correct restatement of what the method
computes, written in fp64 numpy from the definitions:

* ``logprob``  -- tempered softmax statistics, the top-p nucleus (sort based,
  keep-all-ties), truncated/renormalised log-probability and entropy
  (pages: Qwen3-8B VIME train-rollout consistency, "ROCm MI300X and gfx942";
  RL-Kernel ROCm sparse performance page, quick-start command paragraph).
* ``sampling`` -- seeded Gumbel-max draw of a target from the nucleus (test
  inputs), and the definition the GPU sampler follows (``sample_row``).
* ``philox``   -- the Philox-4x32-10 counter-based generator the sampler draws
  its uniforms from (published definition, Salmon et al., SC 2011).
* ``fused``    -- the LM-head forms: logits = hidden . W^T in fp64, then the
  same statistics; the backward through them (prime-rl v0.10.0 release notes,
  "1. Trainer Performance": chunked loss; consistency page, "Canonical
  topology strategy": the loss seed is normalised before model derivatives).
* ``support``  -- the same statistics over a caller-supplied retained set (CSR),
  and whether that set is a valid nucleus (consistency page, "ROCm MI300X
  and gfx942": the sampler's retained set is scored by the logprob kernel).
* ``grpo``     -- group-normalised advantages and the DAPO-style token loss with
  a TIS-truncated ratio and k3 KL (LumenRL README, "Key Features" and
  "Rollout Correction"; RL-Kernel quick-start command: KL coefficient).

It shares no code with the HIP path. Inputs come from ``synth`` (seeded
random numbers only). Every function is pinned by CPU tests against closed
forms, library routines, brute force and finite differences (tests/test_oracle_*.py).
"""
from . import logprob, philox, sampling, fused, grpo, support  # noqa: F401
