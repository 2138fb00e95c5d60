"""GPU parity of rlk_sample_top_p (the rollout-side top-p sampler) against the
oracle's definition (oracle.sampling.sample_row: Gumbel-max over the tempered
nucleus with Philox-4x32-10 uniforms), plus the law of the draws, bitwise
agreement of the returned logprobs with the logits-in scorer, determinism and
batch invariance.

The draw is an argmax of fp64 scores; both sides form them in fp64 from the
same uniforms, so the ids agree except where two scores lie within the
last-bit differences of the two log implementations (accepted when the
oracle's two best scores are within 1e-12 relative), or on rows within 1e-6
of the top-p boundary, where the draw under either valid nucleus passes.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import logprob as OL
from oracle import philox as OP
from oracle import sampling as OS
import grpo_loss_rlk_amd as rlk

from gpu_util import DEV, bf16_to_device, bits_equal, f32_to_device, host

pytestmark = pytest.mark.gpu

SEED, OFFSET = 0x5EED_0123_4567_89AB, 3


def _acceptable(z, T, p, seed, offset, key):
    """Ids a correct sampler may return for this row."""
    z = np.asarray(z, dtype=np.float64)
    if np.isnan(z).any() or np.isposinf(z).any() or not (z > -np.inf).any():
        return {-1}
    keep, _, _, _, alts = OL.nucleus(z, T, p)
    u = OP.row_uniforms(seed, offset, key, z.size)
    ok = set()
    for k in [keep] + alts:
        s = np.full(z.size, -np.inf)
        s[k] = z[k] / T - np.log(-np.log(u[k]))
        order = np.argsort(-s, kind="stable")
        ok.add(int(order[0]))
        if s[order[1]] > -np.inf and s[order[0]] - s[order[1]] <= 1e-12 * abs(s[order[0]]):
            ok.add(int(order[1]))
    return ok


def _draw(x, T, p, seed=SEED, offset=OFFSET, keys=None):
    print(f"  rlk_sample_top_p shape={tuple(x.shape)} T={T} p={p} offset={offset}", flush=True)
    out = rlk.sample_top_p(x, T, p, seed, offset, row_keys=keys)
    torch.cuda.synchronize()
    return out


def _check_ids(ids, z, T, p, seed=SEED, offset=OFFSET, keys=None):
    ids = host(ids)
    exact = 0
    for n in range(len(ids)):
        key = n if keys is None else int(keys[n])
        want = OS.sample_row(z[n], T, p, seed, offset, key)
        if ids[n] == want:
            exact += 1
            continue
        assert ids[n] in _acceptable(z[n], T, p, seed, offset, key), (n, ids[n], want)
    return exact


@pytest.mark.parametrize("name,N,V", [("tiny", 256, 8192), ("qwen", 96, 32768)])
def test_draws_match_the_oracle(name, N, V):
    w = synth.workload(name, N=N, V=V)
    arr = synth.logits_rows(w, range(N))
    z = OL.widen_bf16(arr) if w.dtype == "bf16" else arr.astype(np.float64)
    x = bf16_to_device(arr) if w.dtype == "bf16" else f32_to_device(arr)
    T, p = OL.f32(w.temperature), OL.f32(w.top_p)
    out = _draw(x, w.temperature, w.top_p)
    exact = _check_ids(out["samples"], z, T, p)
    assert exact >= N - 2, exact
    # the returned scores are the logits-in kernel's, bitwise
    ref = rlk.logprob_from_logits(x, out["samples"], w.temperature, w.top_p)
    torch.cuda.synchronize()
    assert bits_equal(out["logprob"], ref["lp_trunc"])
    assert bits_equal(out["entropy"], ref["entropy_trunc"])
    assert bits_equal(out["nucleus_size"], ref["nucleus_size"])
    assert torch.equal(out["flags"], ref["flags"])
    assert not torch.any(out["flags"] & rlk.FLAG_OUTSIDE)        # drawn from the nucleus


def test_edge_rows():
    """p = 1 (whole vocabulary), a tiny p (the argmax, or one of a tied top
    group), -inf entries never drawn, NaN / all -inf rows give -1."""
    r = np.random.default_rng(1)
    V = 3000
    z = r.normal(0, 2, (8, V)).astype(np.float32)
    z[2, [5, 9]] = z[2].max() + 1.0                 # tied top pair
    z[3, ::2] = -np.inf                             # every even id impossible
    z[4, 17] = np.nan
    z[5, :] = -np.inf
    x = f32_to_device(z)
    z64 = z.astype(np.float64)
    for T, p in ((1.0, 1.0), (0.7, 1e-6), (1.3, 0.5)):
        out = _draw(x, T, p)
        ids = host(out["samples"])
        _check_ids(out["samples"], z64, OL.f32(T), OL.f32(p))
        assert ids[4] == -1 and ids[5] == -1
        assert ids[3] % 2 == 1
        if p < 1e-3:
            assert ids[0] == int(np.argmax(z[0])) and ids[2] in (5, 9)
        # every row, the NaN and all -inf ones included, scored bitwise as the
        # logits-in entry point scores targets = samples
        ref = rlk.logprob_from_logits(x, out["samples"], T, p)
        torch.cuda.synchronize()
        assert bits_equal(out["logprob"], ref["lp_trunc"])
        assert bits_equal(out["entropy"], ref["entropy_trunc"])
        assert bits_equal(out["nucleus_size"], ref["nucleus_size"])
        assert torch.equal(out["flags"], ref["flags"])


def test_law_of_the_draws():
    """4096 draws from one row (distinct row keys): frequencies follow the
    tempered softmax renormalised over the nucleus (5 standard deviations)."""
    V, N = 40, 4096
    base = np.linspace(2.0, -3.0, V).astype(np.float32)
    x = f32_to_device(np.tile(base, (N, 1)))
    T, p = 0.8, 0.9
    out = _draw(x, T, p, keys=np.arange(N) * 7919 + 11)
    ids = host(out["samples"])
    keep = OL.nucleus(base.astype(np.float64), OL.f32(T), OL.f32(p))[0]
    q = np.zeros(V)
    e = np.exp((base[keep].astype(np.float64) - base.max()) / OL.f32(T))
    q[keep] = e / e.sum()
    counts = np.bincount(ids, minlength=V)
    assert np.all(counts[~keep] == 0)
    sd = np.sqrt(N * q * (1 - q)) + 1e-9
    assert np.all(np.abs(counts - N * q) <= 5 * sd), (counts, N * q)


def test_determinism_offsets_and_batch_invariance():
    w = synth.workload("qwen", N=300, V=20000)
    arr = synth.logits_rows(w, range(w.N))
    x = bf16_to_device(arr)
    keys = np.arange(w.N, dtype=np.int64) * 3 + 1000
    a = _draw(x, w.temperature, w.top_p, keys=keys)
    b = _draw(x, w.temperature, w.top_p, keys=keys)
    for k in a:
        assert bits_equal(a[k], b[k]) if a[k].dtype != torch.int64 else torch.equal(a[k], b[k]), k
    c = _draw(x, w.temperature, w.top_p, offset=OFFSET + 1, keys=keys)
    assert not torch.equal(a["samples"], c["samples"])          # a new offset, new draws
    for split in (1, 150, 299):
        lo = _draw(x[:split], w.temperature, w.top_p, keys=keys[:split])
        hi = _draw(x[split:], w.temperature, w.top_p, keys=keys[split:])
        assert torch.equal(a["samples"], torch.cat([lo["samples"], hi["samples"]])), split
        assert bits_equal(a["logprob"], torch.cat([lo["logprob"], hi["logprob"]])), split


def test_qwen_logits_full_size_sampled_rows():
    """Config-2 shape (4096 x 151936 bf16, T=0.7, p=0.95) in one call; 8 rows
    against the oracle, every row drawn from its nucleus."""
    w = synth.workload("qwen")
    arr = synth.logits_rows(w, range(w.N))
    x = bf16_to_device(arr)
    out = _draw(x, w.temperature, w.top_p)
    ids = host(out["samples"])
    assert np.all((ids >= 0) & (ids < w.V))
    assert not torch.any(out["flags"] & (rlk.FLAG_OUTSIDE | rlk.FLAG_BAD_TARGET))
    rows = np.random.default_rng(7).choice(w.N, 8, replace=False)
    z = OL.widen_bf16(arr[rows])
    T, p = OL.f32(w.temperature), OL.f32(w.top_p)
    for i, n in enumerate(rows):
        want = OS.sample_row(z[i], T, p, SEED, OFFSET, int(n))
        assert ids[n] == want or ids[n] in _acceptable(z[i], T, p, SEED, OFFSET, int(n)), n


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 2, 9])
def test_tiny_vocabularies_and_zero_rows(dtype, V):
    """V = 1 always draws token 0 with logprob 0; tiny rows agree with the
    oracle's draw; a zero-row call returns empty outputs."""
    r = np.random.default_rng(40 + V)
    z = r.normal(0, 2, (16, V)).astype(np.float32)
    z[1, :] = 0.5                                    # a tied row
    if dtype == "bf16":
        bits = synth.bf16_bits_from_f32(z).reshape(z.shape)
        x, z64 = bf16_to_device(bits), OL.widen_bf16(bits)
    else:
        x, z64 = f32_to_device(z), z.astype(np.float64)
    for T, p in ((1.0, 1.0), (0.7, 0.5)):
        out = _draw(x, T, p)
        _check_ids(out["samples"], z64, OL.f32(T), OL.f32(p))
        if V == 1:
            assert torch.all(out["samples"] == 0) and torch.all(out["logprob"] == 0)
    empty = x[:0]
    out = _draw(empty, 0.7, 0.95)
    assert all(v is None or v.numel() == 0 for v in out.values())


def test_maximum_vocabulary():
    """A bf16 row of 2^24 - 3 tokens (the largest vocabulary the boundary
    accepts, less a ragged tail inside the last 16-byte vector); the draw
    against the oracle's."""
    V = (1 << 24) - 3
    r = np.random.default_rng(55)
    bits = synth.bf16_bits_from_f32(r.normal(0, 2.5, (1, V)).astype(np.float32)).reshape(1, V)
    out = _draw(bf16_to_device(bits), 0.7, 0.95)
    print(f"  oracle draw over {V} tokens", flush=True)
    _check_ids(out["samples"], OL.widen_bf16(bits), OL.f32(0.7), OL.f32(0.95))
