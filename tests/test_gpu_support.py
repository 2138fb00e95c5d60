"""GPU parity of rlk_logprob_from_support (retained-set scoring) against the
fp64 oracle, with edge cases, the nucleus check, and bitwise determinism and
batch invariance.

Tolerance for both dtypes (the logits are read exactly; each mass is fp32 to
about 1 ulp and the sums are fp64, so log Z_S carries about 2.4e-7 relative):
|d lp| <= 1e-5, |d H| <= 1e-5 + 1e-5 |H|; flags exact, except that on rows the
oracle flags as within 1e-6 of the top-p boundary the mismatch bit may go
either way (the GPU nucleus may be the other valid one), and the boundary
bit itself is advisory.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import logprob as OL
from oracle import sampling as OS
from oracle import support as OSup
import grpo_loss_rlk_amd as rlk

from gpu_util import DEV, assert_close_rows, bf16_to_device, bits_equal, f32_to_device, host

pytestmark = pytest.mark.gpu

LP_TOL, H_ATOL, H_RTOL = 1e-5, 1e-5, 1e-5


def _widen(arr, dtype):
    return OL.widen_bf16(arr) if dtype == "bf16" else np.asarray(arr, dtype=np.float64)


def _dev(arr, dtype):
    return bf16_to_device(arr) if dtype == "bf16" else f32_to_device(arr)


def _run(x, y, T, offsets, ids, check_p=0.0):
    print(f"  rlk_logprob_from_support shape={tuple(x.shape)} nnz={len(ids)} T={T} "
          f"check={check_p}", flush=True)
    out = rlk.logprob_from_support(x, torch.as_tensor(y), T, torch.as_tensor(offsets),
                                   torch.as_tensor(ids), check_top_p=check_p)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def _check(g, o, check=False):
    assert_close_rows(g["logprob"], o.lp, LP_TOL, what="logprob")
    assert_close_rows(g["entropy"], o.h, H_ATOL, H_RTOL, what="entropy")
    # with the check, the boundary bit is advisory (the GPU's fixed-point masses
    # and the oracle's fp64 ones may sit on either side of 1e-6) and the
    # mismatch bit is compared on rows the oracle does not flag as boundary
    mask = 0xff if not check else ~(OSup.FLAG_MISMATCH | OSup.FLAG_BOUNDARY) & 0xff
    np.testing.assert_array_equal(g["flags"] & mask, o.flags & mask, err_msg="flags")
    if check:
        firm = (o.flags & OSup.FLAG_BOUNDARY) == 0
        np.testing.assert_array_equal(g["flags"][firm] & OSup.FLAG_MISMATCH,
                                      o.flags[firm] & OSup.FLAG_MISMATCH, err_msg="mismatch")


def _nucleus_inputs(w, rows, T, p):
    arr = synth.logits_rows(w, rows)
    z = _widen(arr, w.dtype)
    masks = np.array([OL.nucleus(z[i], T, p)[0] for i in range(len(rows))])
    y = np.array([OS.gumbel_max_target(z[i], T, p, synth.gumbel_uniforms(w, r, w.V))
                  for i, r in enumerate(rows)], dtype=np.int64)
    return arr, z, masks, y


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nucleus_supports(dtype):
    """Each row's support is its top-p nucleus (oracle): the outputs are the
    truncated ones, and the nucleus check finds no mismatch."""
    if dtype == "f32":
        w = synth.workload("tiny")
    else:
        w = synth.workload("qwen", N=96, V=32768)
    T, p = OL.f32(w.temperature), OL.f32(w.top_p)
    rows = range(w.N)
    arr, z, masks, y = _nucleus_inputs(w, rows, T, p)
    y[3] = int(np.argmin(z[3]))          # outside the nucleus
    y[5] = -1                            # out of range
    offsets, ids = OSup.csr_from_masks(masks)
    x = _dev(arr, w.dtype)
    for check_p in (0.0, p):
        g = _run(x, y, w.temperature, offsets, ids, check_p)
        o = OSup.logprob_from_support(z, y, T, offsets, ids, check_p or None)
        _check(g, o, check=check_p > 0)
    r = OL.logprob_from_logits(z, y, T, p)
    ok = (r.flags & OL.FLAG_BOUNDARY) == 0
    assert_close_rows(g["logprob"][ok], r.lp_trunc[ok], LP_TOL, what="vs truncated lp")


def test_random_supports_and_full_vocab():
    w = synth.workload("qwen", N=64, V=20000)
    T = OL.f32(w.temperature)
    arr = synth.logits_rows(w, range(w.N))
    z = _widen(arr, "bf16")
    r = np.random.default_rng(3)
    masks = r.random((w.N, w.V)) < r.uniform(0.0005, 0.6, (w.N, 1))
    masks[:, 7] = True
    masks[0] = True                      # the full vocabulary
    offsets, ids = OSup.csr_from_masks(masks)
    y = r.integers(0, w.V, w.N)
    y[1] = 7
    g = _run(bf16_to_device(arr), y, w.temperature, offsets, ids)
    _check(g, OSup.logprob_from_support(z, y, T, offsets, ids))
    # full vocabulary = the full-softmax outputs of the logits-in oracle
    full = OL.row(z[0], int(y[0]), T, 1.0)
    assert abs(g["logprob"][0] - full.lp_full) <= LP_TOL
    assert abs(g["entropy"][0] - full.h_full) <= H_ATOL + H_RTOL * abs(full.h_full)


def test_edge_rows():
    """Invalid supports (empty, unsorted, duplicate, out of range, offsets past
    the ids or decreasing), a one-token set, a NaN inside and outside S."""
    V = 300
    z = np.random.default_rng(4).normal(0, 2, (12, V)).astype(np.float32)
    z[8, 40] = np.nan                    # inside row 8's set
    z[9, 41] = np.nan                    # outside row 9's set
    sets = [[], [5, 3], [4, 4, 9], [1, 300], [-1, 2], [17], list(range(V)),
            [2, 50, 299], [10, 40, 50], [10, 50], [0, 1], [6]]
    y = np.array([0, 5, 4, 1, 2, 17, 123, 50, 10, 50, 1, 7], dtype=np.int64)
    lens = np.array([len(s) for s in sets])
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    ids = np.concatenate([np.array(s, dtype=np.int64) for s in sets]).astype(np.int32)
    n_rows = 12
    x = f32_to_device(z)
    g = _run(x, y, 0.9, offsets, ids)
    o = OSup.logprob_from_support(z.astype(np.float64), y, OL.f32(0.9), offsets, ids)
    _check(g, o)
    assert g["flags"][11] & OSup.FLAG_OUTSIDE and np.isneginf(g["logprob"][11])
    assert g["logprob"][5] == 0.0 and g["entropy"][5] == 0.0
    # offsets beyond the ids and decreasing offsets make their rows invalid
    # (nothing past the ids is read)
    off2 = offsets.copy()
    off2[-1] = ids.size + 1000           # the last row runs past the ids
    off2[3] = off2[2] - 1                # row 2 decreasing, row 3 then starts earlier
    g2 = _run(x, y, 0.9, off2, ids)
    assert g2["flags"][11] & OSup.FLAG_BAD_SUPPORT and np.isnan(g2["logprob"][11])
    assert g2["flags"][2] & OSup.FLAG_BAD_SUPPORT
    assert n_rows == len(sets)


def test_mismatch_detection():
    w = synth.workload("tiny", N=32)
    T, p = OL.f32(w.temperature), OL.f32(w.top_p)
    arr, z, masks, y = _nucleus_inputs(w, range(w.N), T, p)
    m2 = masks.copy()
    for n in range(0, w.N, 2):           # even rows: drop the lowest kept / add the next
        kept = np.flatnonzero(masks[n])
        if n % 4 == 0 and kept.size > 1:
            m2[n, kept[np.argmin(z[n, kept])]] = False
        else:
            out = np.flatnonzero(~masks[n])
            m2[n, out[np.argmax(z[n, out])]] = True
    offsets, ids = OSup.csr_from_masks(m2)
    g = _run(f32_to_device(arr), y, w.temperature, offsets, ids, p)
    o = OSup.logprob_from_support(z, y, T, offsets, ids, p)
    _check(g, o, check=True)
    firm = (o.flags & OSup.FLAG_BOUNDARY) == 0
    assert np.all(g["flags"][0::2][firm[0::2]] & OSup.FLAG_MISMATCH)
    assert not np.any(g["flags"][1::2][firm[1::2]] & OSup.FLAG_MISMATCH)
    # p = 1: the whole vocabulary is the nucleus
    full = np.ones((w.N, w.V), dtype=bool)
    offsets, ids = OSup.csr_from_masks(full)
    g = _run(f32_to_device(arr), y, w.temperature, offsets, ids, 1.0)
    assert not np.any(g["flags"] & OSup.FLAG_MISMATCH)


def test_bitwise_determinism_and_batch_invariance():
    w = synth.workload("qwen", N=200, V=32768)
    arr = synth.logits_rows(w, range(w.N))
    r = np.random.default_rng(5)
    masks = r.random((w.N, w.V)) < r.uniform(0.001, 0.5, (w.N, 1))
    masks[:, 0] = True
    offsets, ids = OSup.csr_from_masks(masks)
    y = r.integers(0, w.V, w.N)
    x = bf16_to_device(arr)
    yt = torch.as_tensor(y)

    def call(xx, yy, off, ii):
        out = rlk.logprob_from_support(xx, yy, w.temperature, torch.as_tensor(off),
                                       torch.as_tensor(ii), check_top_p=w.top_p)
        torch.cuda.synchronize()
        return out

    a = call(x, yt, offsets, ids)
    b = call(x, yt, offsets, ids)
    for k in a:
        assert bits_equal(a[k], b[k]), k
    for split in (1, 77, 199):
        lo = call(x[:split], yt[:split], offsets[:split + 1], ids[:offsets[split]])
        hi_off = offsets[split:] - offsets[split]
        hi = call(x[split:], yt[split:], hi_off, ids[offsets[split]:])
        for k in a:
            assert bits_equal(a[k], torch.cat([lo[k], hi[k]])), (k, split)


def test_qwen_logits_full_size_sampled_rows():
    """Config-2 shape (4096 x 151936 bf16) in one call: every row's set is its
    top-k tokens with k ~ U{1..4700} (picked with torch.topk, input
    preparation only); 8 rows against the oracle, and every row finite and
    unflagged."""
    w = synth.workload("qwen")
    arr = synth.logits_rows(w, range(w.N))
    x = bf16_to_device(arr)
    r = np.random.default_rng(6)
    ks = r.integers(1, 4701, w.N)
    top = torch.cat([torch.topk(x[i:i + 256].float(), 4700, dim=1).indices
                     for i in range(0, w.N, 256)]).cpu().numpy()
    sets = [np.sort(top[n, :k]).astype(np.int32) for n, k in enumerate(ks)]
    offsets = np.concatenate([[0], np.cumsum(ks)]).astype(np.int64)
    ids = np.concatenate(sets)
    y = np.array([s[r.integers(0, s.size)] for s in sets], dtype=np.int64)
    g = _run(x, y, w.temperature, offsets, ids)
    rows = r.choice(w.N, 8, replace=False)
    z = OL.widen_bf16(arr[rows])
    sub_off = np.concatenate([[0], np.cumsum(ks[rows])]).astype(np.int64)
    sub_ids = np.concatenate([sets[i] for i in rows])
    o = OSup.logprob_from_support(z, y[rows], OL.f32(w.temperature), sub_off, sub_ids)
    _check({k: v[rows] for k, v in g.items()}, o)
    assert np.all(g["flags"] == 0) and np.all(np.isfinite(g["logprob"]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_maximum_vocabulary(dtype):
    """Rows of 2^24 tokens, the largest vocabulary the boundary accepts: a
    sparse set, the full vocabulary, and the nucleus check on a sparse set."""
    V = 1 << 24
    r = np.random.default_rng(66)
    z32 = r.normal(0, 2.5, (2, V)).astype(np.float32)
    arr = synth.bf16_bits_from_f32(z32).reshape(z32.shape) if dtype == "bf16" else z32
    z = _widen(arr, dtype)
    sparse = np.unique(np.concatenate([[0, V - 1], r.choice(V, 5000, replace=False)]))
    ids = np.concatenate([sparse, np.arange(V)]).astype(np.int32)
    offsets = np.array([0, len(sparse), len(sparse) + V], dtype=np.int64)
    y = np.array([int(sparse[17]), V - 1], dtype=np.int64)
    T = OL.f32(0.7)
    print(f"  oracle support scoring over {V} tokens ({dtype})", flush=True)
    o = OSup.logprob_from_support(z, y, T, offsets, ids)
    g = _run(_dev(arr, dtype), y, 0.7, offsets, ids)
    _check(g, o)
