"""Seeded synthetic inputs for the logprob / entropy / GRPO-loss workloads.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no softmax, no nucleus, no loss): the numbers a method
step itself consumes (the Gumbel uniforms used to pick a target token) are
returned raw, and whoever samples the target does the arithmetic.

Both the GPU tests/bench and the CPU oracle read their inputs from here, so the
two sides consume bit-identical data.

Every array is drawn from numpy's PCG64 through a SeedSequence keyed by
(workload seed, array id, row), so any row can be regenerated on its own
without generating the others.

Workloads (the shapes of the pages' Qwen3-8B GRPO setup: vocabulary 151936,
8 samples per prompt, response cap 6912, 4096 tokens per GPU; and a
Llama-3-70B LM-head shape):

  tiny       N=256 rows, V=8192, fp32 logits ~ N(0, 3^2), T=0.7, p=0.95
  qwen       N=4096, V=151936, bf16 logits ~ N(0, 2.5^2) plus +U(6,12) on
             k ~ U{1..32} distinct 'peak' tokens per row, T=0.7, p=0.95
  fused      hidden bf16 [8192, 4096] ~ N(0,1), W bf16 [151936, 4096]
             ~ N(0, 0.02^2), T=1, p=1, uniform targets
  grpo       32 responses (4 prompts x 8 samples), lengths U{256..6912}
             packed; hidden/W as 'fused'; T=0.7, p=0.95; old/ref logprob
             noise N(0, 0.05^2)/N(0, 0.1^2); rewards Bernoulli(0.5)
  llama70b   hidden bf16 [16384, 8192] ~ N(0,1), W bf16 [128256, 8192]
             ~ N(0, 0.015^2), T=1, p=1, uniform targets
"""
from __future__ import annotations

import dataclasses

import numpy as np

# array ids inside a workload's seed space
_A_LOGITS, _A_PEAKS, _A_GUMBEL, _A_HIDDEN, _A_WEIGHT, _A_TARGET = 1, 2, 3, 4, 5, 6
_A_LENGTHS, _A_REWARD, _A_OLDNOISE, _A_REFNOISE = 7, 8, 9, 10


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    N: int = 0            # rows / tokens
    V: int = 0            # vocabulary
    H: int = 0            # hidden size
    dtype: str = "bf16"   # logits dtype for the logits-in workloads
    sigma: float = 1.0    # logits std (logits-in) or W std (fused)
    temperature: float = 1.0
    top_p: float = 1.0
    # ragged GRPO
    n_prompts: int = 0
    group_size: int = 0
    len_lo: int = 0
    len_hi: int = 0


WORKLOADS = {
    "tiny": Workload("tiny", 1, N=256, V=8192, dtype="f32", sigma=3.0,
                     temperature=0.7, top_p=0.95),
    "qwen": Workload("qwen", 2, N=4096, V=151936, dtype="bf16", sigma=2.5,
                     temperature=0.7, top_p=0.95),
    "fused": Workload("fused", 3, N=8192, V=151936, H=4096, sigma=0.02,
                      temperature=1.0, top_p=1.0),
    "grpo": Workload("grpo", 4, V=151936, H=4096, sigma=0.02,
                     temperature=0.7, top_p=0.95, n_prompts=4, group_size=8,
                     len_lo=256, len_hi=6912),
    "llama70b": Workload("llama70b", 5, N=16384, V=128256, H=8192, sigma=0.015,
                         temperature=1.0, top_p=1.0),
}


def workload(name: str, **overrides) -> Workload:
    """The named workload, optionally with sizes scaled down for tests."""
    return dataclasses.replace(WORKLOADS[name], **overrides)


def _rng(seed: int, array_id: int, row: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, array_id, row])))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 with round-to-nearest-even, as uint16 bit patterns.

    This is the same rounding as torch's ``.to(torch.bfloat16)``; inputs here
    are always finite.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# logits-in workloads
# ----------------------------------------------------------------------------

def peak_ids(w: Workload, row: int) -> tuple[np.ndarray, np.ndarray]:
    """The 'qwen' workload's peak tokens of one row: (ids, added offsets)."""
    r = _rng(w.seed, _A_PEAKS, row)
    k = int(r.integers(1, 33))
    ids = r.choice(w.V, size=min(k, w.V), replace=False)
    add = r.uniform(6.0, 12.0, size=ids.size)
    return ids.astype(np.int64), add


def logits_row_f32(w: Workload, row: int) -> np.ndarray:
    """One row of logits as fp32 (before any bf16 rounding)."""
    z = _rng(w.seed, _A_LOGITS, row).standard_normal(w.V, dtype=np.float32)
    z *= np.float32(w.sigma)
    if w.name == "qwen":
        ids, add = peak_ids(w, row)
        z[ids] = (z[ids].astype(np.float64) + add).astype(np.float32)
    return z


def logits_rows(w: Workload, rows) -> np.ndarray:
    """Logits for the given rows: float32 array (dtype f32) or uint16 bf16 bits."""
    rows = list(rows)
    if w.dtype == "f32":
        out = np.empty((len(rows), w.V), dtype=np.float32)
        for i, r in enumerate(rows):
            out[i] = logits_row_f32(w, r)
        return out
    out = np.empty((len(rows), w.V), dtype=np.uint16)
    for i, r in enumerate(rows):
        out[i] = bf16_bits_from_f32(logits_row_f32(w, r))
    return out


def gumbel_uniforms(w: Workload, row: int, n: int | None = None) -> np.ndarray:
    """Open-interval uniforms u in (0, 1) for one row, one per vocabulary id.

    The Gumbel-max target sampler consumes u[i] for token i.
    """
    n = w.V if n is None else n
    k = _rng(w.seed, _A_GUMBEL, row).integers(0, 1 << 53, size=n, dtype=np.int64)
    return (k.astype(np.float64) + 0.5) * (1.0 / (1 << 53))


def peak_targets(w: Workload, rows) -> np.ndarray:
    """A target id per row: the row's peak token with the largest added offset.

    A generator-only rule (no softmax arithmetic) for runs that need a
    plausible, usually in-nucleus target without sampling it.
    """
    rows = list(rows)
    out = np.empty(len(rows), dtype=np.int64)
    for i, r in enumerate(rows):
        ids, add = peak_ids(w, r)
        out[i] = ids[int(np.argmax(add))]
    return out


# ----------------------------------------------------------------------------
# fused LM-head workloads
# ----------------------------------------------------------------------------

def _normal_bf16_rows(seed: int, array_id: int, rows, cols: int, sigma: float) -> np.ndarray:
    rows = list(rows)
    out = np.empty((len(rows), cols), dtype=np.uint16)
    for i, r in enumerate(rows):
        x = _rng(seed, array_id, r).standard_normal(cols, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[i] = bf16_bits_from_f32(x)
    return out


def hidden_rows(w: Workload, rows) -> np.ndarray:
    """Hidden-state rows, bf16 bits [len(rows), H], ~ N(0, 1)."""
    return _normal_bf16_rows(w.seed, _A_HIDDEN, rows, w.H, 1.0)


def weight_rows(w: Workload, rows) -> np.ndarray:
    """LM-head weight rows (vocabulary ids), bf16 bits [len(rows), H], ~ N(0, sigma^2)."""
    return _normal_bf16_rows(w.seed, _A_WEIGHT, rows, w.H, w.sigma)


def uniform_targets(w: Workload, n: int) -> np.ndarray:
    """Target ids uniform in [0, V)."""
    return _rng(w.seed, _A_TARGET).integers(0, w.V, size=n, dtype=np.int64)


# ----------------------------------------------------------------------------
# ragged GRPO workload
# ----------------------------------------------------------------------------

def response_lengths(w: Workload) -> np.ndarray:
    """Lengths of the n_prompts * group_size responses, uniform in [len_lo, len_hi]."""
    b = w.n_prompts * w.group_size
    return _rng(w.seed, _A_LENGTHS).integers(w.len_lo, w.len_hi + 1, size=b, dtype=np.int64)


def cu_seqlens(lengths: np.ndarray) -> np.ndarray:
    """Packed offsets [B+1] of consecutive responses."""
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum(lengths)
    return out


def rewards(w: Workload) -> np.ndarray:
    """Bernoulli(0.5) reward per response, as float32 0/1."""
    b = w.n_prompts * w.group_size
    return (_rng(w.seed, _A_REWARD).random(b) < 0.5).astype(np.float32)


def logprob_noise(w: Workload, n_tokens: int) -> tuple[np.ndarray, np.ndarray]:
    """Noise added to the new logprobs to make 'old' (sd 0.05) and 'ref' (sd 0.1)."""
    old = _rng(w.seed, _A_OLDNOISE).standard_normal(n_tokens) * 0.05
    ref = _rng(w.seed, _A_REFNOISE).standard_normal(n_tokens) * 0.1
    return old, ref
