"""The seeded generators: determinism, per-row independence and the bf16 cast."""
import hashlib

import numpy as np
import torch

import synth


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_rows_are_independent_and_deterministic():
    w = synth.workload("qwen", V=4096)
    full = synth.logits_rows(w, range(8))
    assert _h(full) == _h(synth.logits_rows(w, range(8)))
    np.testing.assert_array_equal(full[5:6], synth.logits_rows(w, [5]))
    assert full.dtype == np.uint16 and full.shape == (8, 4096)


def test_bf16_cast_matches_torch():
    x = np.random.default_rng(0).normal(0, 3, 100000).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -2.00390625, 3.0e-39]   # exact ties, a denormal
    ours = synth.bf16_bits_from_f32(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    np.testing.assert_array_equal(synth.f32_from_bf16_bits(ours),
                                  torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_peaks_and_targets():
    w = synth.workload("qwen", V=2048)
    for r in range(20):
        ids, add = synth.peak_ids(w, r)
        assert 1 <= ids.size <= 32 and len(set(ids.tolist())) == ids.size
        assert np.all((add >= 6) & (add < 12))
    t = synth.peak_targets(w, range(20))
    assert all(t[r] in synth.peak_ids(w, r)[0] for r in range(20))
    u = synth.gumbel_uniforms(w, 3)
    assert u.size == 2048 and np.all((u > 0) & (u < 1))


def test_ragged_lengths():
    w = synth.workload("grpo")
    L = synth.response_lengths(w)
    assert L.size == 32 and L.min() >= 256 and L.max() <= 6912
    cu = synth.cu_seqlens(L)
    assert cu[0] == 0 and cu[-1] == L.sum() and np.all(np.diff(cu) == L)
    r = synth.rewards(w)
    assert set(np.unique(r).tolist()) <= {0.0, 1.0}
