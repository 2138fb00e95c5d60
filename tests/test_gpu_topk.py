"""GPU parity of the opt-in top-k (then top-p) rule, and of the sampler's
per-row temperature, top-p and top-k, against the fp64 oracle.

Top-k keeps every token whose logit is at least the k-th largest finite one
(ties kept), then top-p runs on the distribution renormalised over that set.
Each row kernel is covered: bf16 rows with V >= 16384 (counting kernel), bf16
rows with V < 16384 and rows handed on from the counting kernel (generic
kernel), fp32 rows (fp32 kernel, and its generic fallback on a crossing bin
of more than 8192 equal values). Tolerances as for the logits-in path: nucleus
size exact except on rows the oracle flags as within 1e-6 of the top-p
boundary (either valid set passes); the threshold exact (it is a logit of the
row: v_k at top-p 1)."""
import numpy as np
import pytest
import torch

import synth
from oracle import fused as OF
from oracle import logprob as OL
from oracle import philox as OP
from oracle import sampling as OS
from oracle import support as OSup
import grpo_loss_rlk_amd as rlk

from gpu_util import DEV, assert_close_rows, bf16_to_device, bits_equal, f32_to_device, host

pytestmark = pytest.mark.gpu

F32_TOL = dict(lp_atol=1e-5, h_atol=1e-5, h_rtol=1e-5)
BF16_TOL = dict(lp_atol=2e-3, h_atol=1e-5, h_rtol=1e-3)


def check(g, o, lp_atol, h_atol, h_rtol, ok_rows=None):
    """GPU outputs g (dict of host arrays) against oracle BatchResult o."""
    rows = np.arange(len(o.lp_full)) if ok_rows is None else np.flatnonzero(ok_rows)
    assert_close_rows(g["lp_full"][rows], o.lp_full[rows], lp_atol, what="lp_full")
    assert_close_rows(g["entropy_full"][rows], o.h_full[rows], h_atol, h_rtol, what="entropy_full")
    bnd = (o.flags & OL.FLAG_BOUNDARY) != 0
    size, lpt, ht = o.size.astype(np.float64), o.lp_trunc.copy(), o.h_trunc.copy()
    for n in np.flatnonzero(bnd):
        for (s2, l2, h2) in o.alts[n]:
            if g["nucleus_size"][n] == s2:
                size[n], lpt[n], ht[n] = s2, l2, h2
    np.testing.assert_array_equal(g["nucleus_size"][rows], size[rows], err_msg="nucleus size")
    assert_close_rows(g["lp_trunc"][rows], lpt[rows], lp_atol, what="lp_trunc")
    assert_close_rows(g["entropy_trunc"][rows], ht[rows], h_atol, h_rtol, what="entropy_trunc")
    nb = rows[~bnd[rows] & ~np.isnan(o.tau[rows])]
    np.testing.assert_array_equal(g["threshold"][nb], o.tau[nb].astype(np.float32), err_msg="tau")
    outside = np.isneginf(g["lp_trunc"][rows]) & ~np.isnan(g["lp_full"][rows])
    np.testing.assert_array_equal((g["flags"][rows] & OL.FLAG_OUTSIDE) != 0, outside,
                                  err_msg="outside")


def run(x, y, T, p, **kw):
    print(f"  rlk_logprob_from_logits top-k shape={tuple(x.shape)} T={T} p={p} "
          f"k={kw.get('top_k', 'per row')}", flush=True)
    out = rlk.logprob_from_logits(x, torch.as_tensor(y), T, p, **kw)
    torch.cuda.synchronize()
    return {k: (None if v is None else host(v)) for k, v in out.items()}


@pytest.mark.parametrize("V", [151936, 4000])
@pytest.mark.parametrize("k,p", [(1, 1.0), (20, 0.95), (20, 1.0), (300, 0.95), (5000, 0.9)])
def test_bf16_top_k(V, k, p):
    """bf16 rows (counting kernel at V = 151936, generic kernel at 4000),
    the pages' distribution with peaks; in-nucleus and random targets."""
    w = synth.workload("qwen", V=V)
    N = 48
    arr = synth.logits_rows(w, range(N))
    z = OL.widen_bf16(arr)
    y = synth.peak_targets(w, range(N))
    y[::3] = np.random.default_rng(k).integers(0, V, (N + 2) // 3)
    g = run(bf16_to_device(arr), y, 0.7, p, top_k=k)
    o = OL.logprob_from_logits(z, y, OL.f32(0.7), OL.f32(p), k)
    check(g, o, **BF16_TOL)
    if k < 50:
        assert np.all(g["nucleus_size"] >= 1) and np.any(g["nucleus_size"] < k + 200)


@pytest.mark.parametrize("k,p", [(1, 1.0), (40, 0.95), (40, 1.0), (2000, 0.95)])
def test_f32_top_k(k, p):
    w = synth.workload("tiny")
    N = 64
    arr = synth.logits_rows(w, range(N))
    z = arr.astype(np.float64)
    y = np.random.default_rng(k).integers(0, w.V, N)
    g = run(f32_to_device(arr), y, 0.7, p, top_k=k)
    o = OL.logprob_from_logits(z, y, OL.f32(0.7), OL.f32(p), k)
    check(g, o, **F32_TOL)


def test_per_row_top_k_and_parameters():
    """Per-row k (0, 1, within the row, at and above V, negative), with
    per-row temperature and top-p; a negative k gives NaN outputs and the
    bad-parameter flag."""
    for dtype, V in (("bf16", 151936), ("bf16", 4000), ("f32", 8192)):
        w = synth.workload("qwen" if dtype == "bf16" else "tiny", V=V)
        N = 40
        arr = synth.logits_rows(w, range(N))
        z = OL.widen_bf16(arr) if dtype == "bf16" else arr.astype(np.float64)
        x = bf16_to_device(arr) if dtype == "bf16" else f32_to_device(arr)
        r = np.random.default_rng(V)
        ks = r.integers(1, 400, N).astype(np.int32)
        ks[0], ks[1], ks[2], ks[3], ks[4] = 0, 1, V, V + 7, -3
        Ts = r.choice([0.5, 0.7, 1.0, 1.6], N).astype(np.float32)
        ps = r.choice([0.5, 0.9, 0.95, 1.0], N).astype(np.float32)
        y = np.argmax(z, axis=1)
        g = run(x, y, 0.7, 0.95, temperature_per_row=Ts, top_p_per_row=ps, top_k_per_row=ks)
        assert g["flags"][4] & rlk.FLAG_BAD_PARAM and np.isnan(g["lp_trunc"][4])
        good = ks >= 0
        o = OL.logprob_from_logits(z, y, Ts.astype(np.float64), ps.astype(np.float64),
                                   np.maximum(ks, 0))
        check(g, o, **(BF16_TOL if dtype == "bf16" else F32_TOL), ok_rows=good)
        # k = 0 and k >= V: the plain top-p rule
        plain = run(x[:4].contiguous(), y[:4], 0.7, 0.95, temperature_per_row=Ts[:4],
                    top_p_per_row=ps[:4])
        for n in (0, 2, 3):
            assert g["nucleus_size"][n] == plain["nucleus_size"][n]


def test_hand_offs_and_crossing_bin_fallback():
    """bf16 rows the counting kernel hands on (a value below its window) and an
    fp32 row whose crossing bin holds 20000 equal values (the fp32 kernel's
    generic fallback), with top-k."""
    w = synth.workload("qwen", V=32768)
    arr = synth.logits_rows(w, range(8)).copy()
    arr[:, 100] = 0x0001                   # |z| far below the counted window: handed on
    y = synth.peak_targets(w, range(8))
    for k, p in ((10, 0.95), (3000, 1.0)):
        g = run(bf16_to_device(arr), y, 0.7, p, top_k=k)
        check(g, OL.logprob_from_logits(OL.widen_bf16(arr), y, OL.f32(0.7), OL.f32(p), k),
              **BF16_TOL)
    z = np.random.default_rng(3).normal(0, 1, (2, 30000)).astype(np.float32)
    z[:, :20000] = 0.25                    # one value x 20000 dominates the crossing bin
    z[:, 20000:20010] = 3.0
    for k, p in ((15000, 0.9), (20005, 0.99), (5, 0.5)):
        yy = np.array([0, 20001])
        g = run(f32_to_device(z), yy, 1.0, p, top_k=k)
        check(g, OL.logprob_from_logits(z.astype(np.float64), yy, 1.0, OL.f32(p), k), **F32_TOL)


def test_bitwise_and_batch_invariant():
    w = synth.workload("qwen")
    G = torch.cuda.get_device_properties(0).multi_processor_count
    N = 2 * G + 3
    arr = synth.logits_rows(w, range(7))
    idx = np.arange(N) % 7
    x = bf16_to_device(arr[idx])
    y = torch.as_tensor(synth.peak_targets(w, range(7))[idx])
    a = rlk.logprob_from_logits(x, y, 0.7, 0.95, top_k=64)
    b = rlk.logprob_from_logits(x, y, 0.7, 0.95, top_k=64)
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k
            v = host(a[k])
            for c in range(7):
                pos = np.flatnonzero(idx == c)
                assert all(v[q].tobytes() == v[pos[0]].tobytes() for q in pos), (k, c)


# ------------------------------------------------------------------ sampler

SEED, OFFSET = 0x0DDB_A11_5EED, 11


def _acceptable(z, T, p, k, key):
    z = np.asarray(z, dtype=np.float64)
    if np.isnan(z).any() or np.isposinf(z).any() or not (z > -np.inf).any():
        return {-1}
    keep, _, _, _, alts = OL.nucleus(z, T, p, k)
    u = OP.row_uniforms(SEED, OFFSET, key, z.size)
    ok = set()
    for s_ in [keep] + alts:
        s = np.full(z.size, -np.inf)
        s[s_] = z[s_] / T - np.log(-np.log(u[s_]))
        order = np.argsort(-s, kind="stable")
        ok.add(int(order[0]))
        if s[order[1]] > -np.inf and s[order[0]] - s[order[1]] <= 1e-12 * abs(s[order[0]]):
            ok.add(int(order[1]))
    return ok


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("bf16", 4000), ("f32", 8192)])
def test_sampler_per_row_parameters_and_top_k(dtype, V):
    """Per-row temperature, top-p and top-k (one negative k: no draw, the
    bad-parameter flag); the draws equal the oracle's, and the returned
    logprob, entropy and nucleus size are bitwise the scorer's for
    targets = samples with the same per-row parameters."""
    w = synth.workload("qwen" if dtype == "bf16" else "tiny", V=V)
    N = 64
    arr = synth.logits_rows(w, range(N))
    z = OL.widen_bf16(arr) if dtype == "bf16" else arr.astype(np.float64)
    x = bf16_to_device(arr) if dtype == "bf16" else f32_to_device(arr)
    r = np.random.default_rng(V + 1)
    Ts = r.choice([0.4, 0.7, 1.0, 1.3], N).astype(np.float32)
    ps = r.choice([0.6, 0.9, 0.95, 1.0], N).astype(np.float32)
    ks = r.choice([0, 1, 5, 50, 600], N).astype(np.int32)
    ks[7] = -1
    Ts[9] = 0.0                             # out of range: no draw
    print(f"  rlk_sample_top_p per-row parameters dtype={dtype} V={V}", flush=True)
    out = rlk.sample_top_p(x, 0.7, 0.95, SEED, OFFSET, temperature_per_row=Ts,
                           top_p_per_row=ps, top_k_per_row=ks)
    torch.cuda.synchronize()
    ids = host(out["samples"])
    fl = host(out["flags"])
    for n in (7, 9):
        assert ids[n] == -1 and fl[n] & rlk.FLAG_BAD_PARAM
    exact = 0
    for n in range(N):
        if n in (7, 9):
            continue
        T, p, k = float(Ts[n]), float(ps[n]), int(ks[n])
        want = OS.sample_row(z[n], T, p, SEED, OFFSET, n, top_k=k)
        if ids[n] == want:
            exact += 1
        else:
            assert ids[n] in _acceptable(z[n], T, p, k, n), (n, ids[n], want)
        keep, *_ = OL.nucleus(z[n], T, p, k)
        assert keep[ids[n]]
    assert exact >= N - 4, exact
    ref = rlk.logprob_from_logits(x, out["samples"], 0.7, 0.95, temperature_per_row=Ts,
                                  top_p_per_row=ps, top_k_per_row=ks)
    torch.cuda.synchronize()
    ok = torch.as_tensor(ids >= 0).to(DEV)
    assert bits_equal(out["logprob"][ok], ref["lp_trunc"][ok])
    assert bits_equal(out["entropy"][ok], ref["entropy_trunc"][ok])
    assert torch.equal(out["nucleus_size"][ok], ref["nucleus_size"][ok])


def test_sampler_law_with_top_k():
    """Over many offsets the draws of one row follow the tempered softmax over
    its top-k/top-p set (5 sd per token) and never leave it."""
    z = np.array([2.0, 1.7, 1.5, 1.5, 1.2, 0.3, -0.2, -1.0, 0.9, 0.95] + [-3.0] * 22,
                 dtype=np.float32)
    T, p, k = 0.8, 0.97, 5
    keep, *_ = OL.nucleus(z.astype(np.float64), T, OL.f32(p), k)
    q = np.zeros(z.size)
    q[keep] = np.exp(z[keep] / T) / np.exp(z[keep] / T).sum()
    draws = 4096
    x = f32_to_device(np.tile(z, (draws, 1)))
    print("  rlk_sample_top_p law with top-k", flush=True)
    out = rlk.sample_top_p(x, T, p, 123, 0, row_keys=np.arange(draws), top_k=k)
    ids = host(out["samples"])
    counts = np.bincount(ids, minlength=z.size).astype(np.float64)
    assert counts[~keep].sum() == 0
    sd = np.sqrt(draws * q * (1 - q)) + 1e-9
    assert np.all(np.abs(counts - draws * q) <= 5 * sd)


# ------------------------------------------------------------- fused and support

@pytest.mark.parametrize("p", [1.0, 0.9])
def test_fused_forward_and_backward_with_top_k(p):
    """The fused LM head with top-k at top-p 1 (logits stored and cut, no
    longer the tile-statistics path) and below; the backward through the
    forward's top-k nucleus (held fixed) against the oracle's."""
    N, H, V, T, k = 300, 128, 3001, 0.8, 40
    w = synth.workload("grpo", N=N, H=H, V=V, sigma=0.15, temperature=T, top_p=p)
    hb = synth.hidden_rows(w, range(N))
    wb = synth.weight_rows(w, range(V))
    h64, w64 = OL.widen_bf16(hb), OL.widen_bf16(wb)
    z64 = OF.logits(h64, w64)
    y = np.argmax(z64, axis=1)
    y[5] = int(np.argmin(z64[5]))           # outside the top-k set
    h, W, yt = bf16_to_device(hb), bf16_to_device(wb), torch.as_tensor(y)
    print(f"  rlk fused top-k N={N} H={H} V={V} k={k} p={p}", flush=True)
    f = rlk.logprob_fused_linear(h, W, yt, T, p, top_k=k)
    torch.cuda.synchronize()
    o = OL.logprob_from_logits(z64, y, OL.f32(T), OL.f32(p), k)
    bnd = (o.flags & OL.FLAG_BOUNDARY) != 0
    assert bnd.mean() < 0.05
    ok = ~bnd
    np.testing.assert_array_equal(host(f["nucleus_size"])[ok], o.size[ok])
    assert np.all(host(f["nucleus_size"])[ok] <= k)
    assert_close_rows(host(f["logprob"])[ok], o.lp_trunc[ok], 2e-3, what="logprob")
    assert_close_rows(host(f["entropy"])[ok], o.h_trunc[ok], 1e-5, 1e-3, what="entropy")
    r = np.random.default_rng(9)
    g_lp = (r.standard_normal(N) / N).astype(np.float32)
    g_h = (r.standard_normal(N) / N).astype(np.float32)
    g_lp[bnd], g_h[bnd] = 0.0, 0.0
    dh, dw = rlk.logprob_fused_linear_bwd(h, W, yt, f["saved"], torch.as_tensor(g_lp).to(DEV),
                                          torch.as_tensor(g_h).to(DEV), T, p, top_k=k)
    torch.cuda.synchronize()
    dh_ref, dw_ref = OF.backward(h64, w64, y, g_lp.astype(np.float64), g_h.astype(np.float64),
                                 OL.f32(T), OL.f32(p), k)
    for got, want in ((host(dh.float()).astype(np.float64), dh_ref),
                      (host(dw).astype(np.float64), dw_ref)):
        assert np.linalg.norm(got - want) <= 5e-3 * np.linalg.norm(want)


def test_support_check_with_top_k():
    """The retained-support check against a top-k/top-p nucleus: the oracle's
    top-k nuclei pass, the plain top-p nuclei (larger here) are mismatches."""
    w = synth.workload("qwen", V=32768)
    N, T, p, k = 24, 0.7, 0.95, 8
    arr = synth.logits_rows(w, range(N))
    z = OL.widen_bf16(arr)
    y = synth.peak_targets(w, range(N))
    x = bf16_to_device(arr)
    mk = np.array([OL.nucleus(z[n], OL.f32(T), OL.f32(p), k)[0] for n in range(N)])
    mp = np.array([OL.nucleus(z[n], OL.f32(T), OL.f32(p))[0] for n in range(N)])
    assert np.any(mp.sum(axis=1) > mk.sum(axis=1))
    for masks, expect_mismatch in ((mk, False), (mp, True)):
        off, ids = OSup.csr_from_masks(masks)
        print(f"  rlk_logprob_from_support top-k check k={k}", flush=True)
        s = rlk.logprob_from_support(x, torch.as_tensor(y), T, torch.as_tensor(off),
                                     torch.as_tensor(ids), check_top_p=p, check_top_k=k)
        o = OSup.logprob_from_support(z, y, OL.f32(T), off, ids, check_p=OL.f32(p), check_k=k)
        fl = host(s["flags"])
        bnd = (o.flags & OSup.FLAG_BOUNDARY) != 0
        np.testing.assert_array_equal((fl[~bnd] & rlk.FLAG_MISMATCH) != 0,
                                      (o.flags[~bnd] & OSup.FLAG_MISMATCH) != 0)
        if expect_mismatch:
            diff = mp.sum(axis=1) != mk.sum(axis=1)
            assert np.all(fl[diff & ~bnd] & rlk.FLAG_MISMATCH)
        else:
            assert not np.any(fl[~bnd] & rlk.FLAG_MISMATCH)
