"""GPU parity of rlk_logprob_from_logits against the fp64 oracle, plus bitwise
determinism and batch invariance.

Tolerances: fp32 logits |d lp| <= 1e-5, |d H| <= 1e-5 + 1e-5 |H|; bf16 logits
(the oracle consumes the same bf16 bits) |d lp| <= 2e-3, |d H| <= 1e-3 |H| with
a 1e-5 floor; nucleus size and membership exact except on rows the oracle
flags as within 1e-6 of the top-p boundary, where either valid set passes.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import logprob as OL
from oracle import sampling as OS
import grpo_loss_rlk_amd as rlk

from gpu_util import DEV, assert_close_rows, bf16_to_device, f32_to_device, host

pytestmark = pytest.mark.gpu

F32_TOL = dict(lp_atol=1e-5, h_atol=1e-5, h_rtol=1e-5)
BF16_TOL = dict(lp_atol=2e-3, h_atol=1e-5, h_rtol=1e-3)


def widen(arr, dtype):
    return OL.widen_bf16(arr) if dtype == "bf16" else np.asarray(arr, dtype=np.float64)


def to_dev(arr, dtype):
    return bf16_to_device(arr) if dtype == "bf16" else f32_to_device(arr)


def run(arr, dtype, targets, T, p, **kw):
    x = to_dev(arr, dtype)
    print(f"  rlk_logprob_from_logits dtype={dtype} shape={tuple(x.shape)} T={T} p={p}", flush=True)
    out = rlk.logprob_from_logits(x, torch.as_tensor(targets), T, p, **kw)
    torch.cuda.synchronize()
    return {k: (None if v is None else host(v)) for k, v in out.items()}


def check(g, o, lp_atol, h_atol, h_rtol, vocab_rows=None):
    """Compare GPU outputs g (dict of arrays) with oracle BatchResult o."""
    N = len(o.lp_full)
    assert_close_rows(g["lp_full"], o.lp_full, lp_atol, what="lp_full")
    assert_close_rows(g["entropy_full"], o.h_full, h_atol, h_rtol, what="entropy_full")
    bnd = (o.flags & OL.FLAG_BOUNDARY) != 0
    size, lpt, ht = o.size.astype(np.float64), o.lp_trunc.copy(), o.h_trunc.copy()
    for n in np.flatnonzero(bnd):                 # pick the valid set the GPU chose
        for (s2, l2, h2) in o.alts[n]:
            if g["nucleus_size"][n] == s2:
                size[n], lpt[n], ht[n] = s2, l2, h2
    np.testing.assert_array_equal(g["nucleus_size"], size, err_msg="nucleus size")
    assert_close_rows(g["lp_trunc"], lpt, lp_atol, what="lp_trunc")
    assert_close_rows(g["entropy_trunc"], ht, h_atol, h_rtol, what="entropy_trunc")
    keep_bits = OL.FLAG_BAD_TARGET | OL.FLAG_NONFINITE
    np.testing.assert_array_equal(g["flags"] & keep_bits, o.flags & keep_bits, err_msg="flags")
    outside = np.isneginf(g["lp_trunc"]) & ~np.isnan(g["lp_full"])
    np.testing.assert_array_equal((g["flags"] & OL.FLAG_OUTSIDE) != 0, outside, err_msg="outside")
    nb = ~bnd & ~np.isnan(o.tau)
    np.testing.assert_array_equal(g["threshold"][nb], o.tau[nb].astype(np.float32), err_msg="tau")


def oracle_targets(w, logits64, rows):
    T, p = OL.f32(w.temperature), OL.f32(w.top_p)
    return np.array([OS.gumbel_max_target(logits64[i], T, p, synth.gumbel_uniforms(w, r, logits64.shape[1]))
                     for i, r in enumerate(rows)], dtype=np.int64)


# --------------------------------------------------------------- workloads

def test_tiny_fp32_full_config():
    """N=256, V=8192 fp32 ~ N(0, 3^2), T=0.7, p=0.95, Gumbel-max targets."""
    w = synth.workload("tiny")
    arr = synth.logits_rows(w, range(w.N))
    z = widen(arr, "f32")
    y = oracle_targets(w, z, range(w.N))
    o = OL.logprob_from_logits(z, y, OL.f32(w.temperature), OL.f32(w.top_p))
    g = run(arr, "f32", y, w.temperature, w.top_p)
    check(g, o, **F32_TOL)
    assert np.all((o.flags & OL.FLAG_OUTSIDE) == 0)        # sampled targets are in the nucleus


@pytest.mark.parametrize("V,N", [(151936, 48), (20003, 37), (16384, 5), (4000, 9)])
def test_qwen_bf16_rows(V, N):
    """bf16 N(0, 2.5^2) + 1..32 peaks per row, T=0.7, p=0.95, Gumbel-max targets."""
    w = synth.workload("qwen", V=V)
    arr = synth.logits_rows(w, range(N))
    z = widen(arr, "bf16")
    y = oracle_targets(w, z, range(N))
    o = OL.logprob_from_logits(z, y, OL.f32(w.temperature), OL.f32(w.top_p))
    g = run(arr, "bf16", y, w.temperature, w.top_p)
    check(g, o, **BF16_TOL)


def test_qwen_full_size_sampled_rows():
    """The full 4096 x 151936 bf16 launch (as the benchmark times it); sampled
    rows checked against the oracle one by one."""
    w = synth.workload("qwen")
    arr = synth.logits_rows(w, range(w.N))
    y = synth.peak_targets(w, range(w.N))
    rows = np.random.default_rng(0).choice(w.N, 24, replace=False)
    z = widen(arr[rows], "bf16")
    y[rows] = oracle_targets(w, z, rows)          # Gumbel-max targets where checked
    g = run(arr, "bf16", y, w.temperature, w.top_p)
    o = OL.logprob_from_logits(z, y[rows], OL.f32(w.temperature), OL.f32(w.top_p))
    check({k: (None if v is None else v[rows]) for k, v in g.items()}, o, **BF16_TOL)
    assert np.all(np.isfinite(g["lp_trunc"][rows]))
    assert np.all(g["nucleus_size"] >= 1) and np.all(g["nucleus_size"] <= w.V)
    outside = (g["flags"] & rlk.FLAG_OUTSIDE) != 0
    np.testing.assert_array_equal(outside, np.isneginf(g["lp_trunc"]))


def test_fp32_long_rows_generic_path():
    w = synth.workload("tiny", V=151936)
    arr = synth.logits_rows(w, range(6))
    z = widen(arr, "f32")
    y = oracle_targets(w, z, range(6))
    o = OL.logprob_from_logits(z, y, OL.f32(0.7), OL.f32(0.95))
    check(run(arr, "f32", y, 0.7, 0.95), o, **F32_TOL)


# --------------------------------------------------------------- edge rows

def _edge_rows(V, dtype):
    rng = np.random.default_rng(123)
    rows, tg = [], []
    base = rng.normal(0, 2.5, V).astype(np.float32)
    rows.append(np.full(V, 0.75, np.float32)); tg.append(3)                 # uniform
    r = np.zeros(V, np.float32); r[7] = 100.0; rows.append(r); tg.append(7)  # one-hot dominant
    r = base.copy(); r[::3] = -np.inf; rows.append(r); tg.append(1)          # -inf entries
    r = base.copy(); r[::3] = -np.inf; rows.append(r); tg.append(3)          # target is -inf
    r = base.copy(); r[5] = np.nan; rows.append(r); tg.append(0)             # NaN
    r = base.copy(); r[9] = np.inf; rows.append(r); tg.append(0)             # +inf
    rows.append(np.full(V, -np.inf, np.float32)); tg.append(0)               # nothing finite
    rows.append(base.copy()); tg.append(V)                                    # target out of range
    rows.append(base.copy()); tg.append(-1)
    r = np.round(base * 2) / 2; rows.append(r.astype(np.float32)); tg.append(int(np.argmax(r)))  # heavy ties
    r = base.copy(); r[:V // 2] = 0.0; r[V // 2:V // 2 + 50] = -0.0; rows.append(r); tg.append(V // 2)  # +-0
    r = np.full(V, -5.0, np.float32); r[:4] = [3, 3, 3, 2]; rows.append(r); tg.append(2)   # tied top group
    arr = np.stack(rows)
    if dtype == "bf16":
        arr = synth.bf16_bits_from_f32(np.where(np.isnan(arr), 0, arr)).reshape(arr.shape)
        arr[4, 5] = 0x7FC0                                                   # bf16 NaN
    return arr, np.array(tg, dtype=np.int64)


@pytest.mark.parametrize("dtype,V", [("f32", 5000), ("f32", 20000), ("bf16", 151936),
                                     ("bf16", 20000), ("bf16", 1000)])
@pytest.mark.parametrize("T,p", [(0.7, 0.95), (1.0, 1.0), (0.2, 1e-6), (1.8, 0.5)])
def test_edge_rows(dtype, V, T, p):
    arr, y = _edge_rows(V, dtype)
    z = widen(arr, dtype)
    o = OL.logprob_from_logits(z, y, OL.f32(T), OL.f32(p))
    g = run(arr, dtype, y, T, p)
    check(g, o, **(F32_TOL if dtype == "f32" else BF16_TOL))


def _window_edge_rows(V):
    """bf16 rows (as 16-bit codes) aimed at the counting kernel's index
    arithmetic: the counters hold magnitudes 0x2000..0x5fff, stored rotated
    (0x4000..0x5fff first), and the row max is located per 16-byte group of
    four magnitudes before the exact one is picked inside the group."""
    rng = np.random.default_rng(2024)
    base = synth.bf16_bits_from_f32(rng.normal(0, 2.5, V).astype(np.float32))
    rows, tg = [], []
    # all negative, no zero: the max is the negative value of smallest magnitude
    r = base | np.uint16(0x8000); r[r == 0x8000] = 0xBF80; rows.append(r); tg.append(int(np.argmin(r & 0x7FFF)))
    # only magnitudes around the rotation seam (|z| near 2), both signs
    r = rng.choice(np.arange(0x3FFC, 0x4004, dtype=np.uint16), V); r[rng.random(V) < 0.5] |= 0x8000
    rows.append(r); tg.append(int(np.argmax(np.where(r & 0x8000, 0, r))))
    # the largest counted magnitude present (|z| about 3.7e19), once and negated
    r = base.copy(); r[[10, 11]] = [0x5FFF, 0xDFFE]; rows.append(r); tg.append(10)
    # the smallest counted magnitudes (|z| about 1e-19) mixed in
    r = base.copy(); r[rng.choice(V, 64, replace=False)] = rng.choice(
        np.array([0x2000, 0x2001, 0x2003, 0xA000, 0xA002], dtype=np.uint16), 64); rows.append(r); tg.append(5)
    # max group holding several present magnitudes: 1.0 .. 1.0234375 (codes 0x3F80..0x3F83)
    r = np.full(V, 0xBF80, np.uint16); r[:8] = [0x3F80, 0x3F81, 0x3F82, 0x3F83, 0x3F81, 0x3F80, 0x3F7F, 0x3F7C]
    rows.append(r); tg.append(3)
    # negatives only, smallest magnitudes inside one group: -0.5 .. -0.50390625 (0xBF00..0xBF01)
    r = np.full(V, 0xC000, np.uint16); r[[3, 4, 5]] = [0xBF01, 0xBF00, 0xBF02]; rows.append(r); tg.append(4)
    return np.stack(rows), np.array(tg, dtype=np.int64)


@pytest.mark.parametrize("V", [151936, 20000])
@pytest.mark.parametrize("T,p", [(0.7, 0.95), (1.0, 1.0), (1.3, 0.5)])
def test_bf16_counter_window_edges(V, T, p):
    arr, y = _window_edge_rows(V)
    zz = widen(arr, "bf16")
    o = OL.logprob_from_logits(zz, y, OL.f32(T), OL.f32(p))
    g = run(arr, "bf16", y, T, p)
    check(g, o, **BF16_TOL)


@pytest.mark.parametrize("T,p", [(0.7, 0.95), (1.0, 1.0), (0.7, 0.3)])
def test_special_values_in_realistic_rows(T, p):
    """Zeros, -0, -inf (vocabulary masking), tiny and huge magnitudes mixed
    into Qwen-shaped rows: every row must match the oracle whichever kernel
    path takes it."""
    w = synth.workload("qwen")
    N = 10
    rows = synth.logits_rows(w, range(N))
    z = synth.f32_from_bf16_bits(rows).copy()
    rng = np.random.default_rng(77)
    y = synth.peak_targets(w, range(N))
    z[0, rng.choice(w.V, 1, replace=False)] = 0.0
    z[1, rng.choice(w.V, 1000, replace=False)] = 0.0
    z[2, rng.choice(w.V, 5, replace=False)] = -np.inf
    z[3, rng.choice(w.V, 20000, replace=False)] = -np.inf
    z[3, rng.choice(w.V, 300, replace=False)] = 0.0
    z[4, rng.choice(w.V, 40, replace=False)] = -0.0
    z[5, 11] = 0.0; y[5] = 11                           # target on a zero
    z[6, 12] = -np.inf; y[6] = 12                       # target masked out
    z[7, rng.choice(w.V, 3, replace=False)] = 1e-30     # below the counted window
    z[8, :] = np.where(z[8] > 0, -z[8], z[8])           # all negative
    z[8, rng.choice(w.V, 2, replace=False)] = 0.0       # ... with zeros at the top
    z[9, rng.choice(w.V, 2, replace=False)] = 3e19      # above the counted window
    arr = synth.bf16_bits_from_f32(np.where(np.isnan(z), 0, z)).reshape(z.shape)
    zz = widen(arr, "bf16")
    o = OL.logprob_from_logits(zz, y, OL.f32(T), OL.f32(p))
    g = run(arr, "bf16", y, T, p)
    check(g, o, **BF16_TOL)


def test_hand_off_from_every_finisher_path():
    """More rows than blocks, so a block post-processes rows both with its
    finisher waves (while the next row streams) and with the whole block
    (its last row). Rows the counting kernel must hand to the generic
    algorithm — a NaN, a +inf, a magnitude above the counted window, and a
    value present more than 65535 times (its 16-bit counter wraps, caught by
    the checksum of all counts) — sit on both paths and on a block's only
    row; every row must match the oracle."""
    w = synth.workload("qwen")
    N, G = 300, 256                       # blocks 0..43 take two rows: b and b + 256
    rows = synth.logits_rows(w, range(N))
    y = synth.peak_targets(w, range(N))
    rows[3, 17] = 0x7FC0                  # NaN, finisher waves (block 3, first of two rows)
    rows[259, 5] = 0x7F80                 # +inf, whole block (block 3, last row)
    rows[100, 9] = 0x6010                 # above the window, a block's only row
    rows[10, :70000] = 0x3F80             # 70000 copies of 1.0, finisher waves (block 10)
    rows[266, :66000] = 0xBF80            # 66000 copies of -1.0, whole block (block 10)
    y[10] = 3
    y[266] = 70000
    zz = widen(rows, "bf16")
    o = OL.logprob_from_logits(zz, y, OL.f32(0.7), OL.f32(0.95))
    g = run(rows, "bf16", y, 0.7, 0.95)
    check(g, o, **BF16_TOL)
    assert G < N < 2 * G


def test_per_row_temperature_and_top_p():
    w = synth.workload("qwen", V=32768)
    N = 16
    arr = synth.logits_rows(w, range(N))
    z = widen(arr, "bf16")
    Ts = np.array([0.2, 0.7, 1.0, 1.8] * 4, dtype=np.float32)
    ps = np.array([1.0, 0.95, 0.5, 1e-6, 0.9, 0.99, 0.3, 0.999] * 2, dtype=np.float32)
    y = np.array([int(np.argmax(z[i])) for i in range(N)], dtype=np.int64)
    o = OL.logprob_from_logits(z, y, Ts.astype(np.float64), ps.astype(np.float64))
    g = run(arr, "bf16", y, 1.0, 1.0, temperature_per_row=Ts, top_p_per_row=ps)
    check(g, o, **BF16_TOL)
    bad = Ts.copy(); bad[3] = 0.0
    g = run(arr, "bf16", y, 1.0, 1.0, temperature_per_row=bad, top_p_per_row=ps)
    assert g["flags"][3] & rlk.FLAG_BAD_PARAM and np.isnan(g["lp_full"][3])


def test_padded_row_stride():
    w = synth.workload("qwen")
    N = 6
    arr = synth.logits_rows(w, range(N))
    pad = np.full((N, 152576), 0x7F80, dtype=np.uint16)      # +inf padding must never be read
    pad[:, :w.V] = arr
    y = synth.peak_targets(w, range(N))
    x = bf16_to_device(pad)
    a = rlk.logprob_from_logits(x, torch.as_tensor(y), 0.7, 0.95, vocab=w.V)
    b = rlk.logprob_from_logits(x[:, :w.V].contiguous(), torch.as_tensor(y), 0.7, 0.95)
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k
    o = OL.logprob_from_logits(widen(arr, "bf16"), y, OL.f32(0.7), OL.f32(0.95))
    check({k: host(v) for k, v in a.items()}, o, **BF16_TOL)


# ------------------------------------------------------- determinism / batch invariance

@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f32", 8192), ("bf16", 4000)])
def test_bitwise_run_to_run_and_batch_invariance(dtype, V):
    name = "tiny" if dtype == "f32" else "qwen"
    w = synth.workload(name, V=V)
    N = 64
    arr = synth.logits_rows(w, range(N))
    y = torch.as_tensor(np.random.default_rng(1).integers(0, V, N))
    x = to_dev(arr, dtype)
    ref = rlk.logprob_from_logits(x, y, 0.7, 0.95)
    again = rlk.logprob_from_logits(x, y, 0.7, 0.95)
    for k in ref:
        if ref[k] is not None:
            assert torch.equal(ref[k], again[k]), k
    for split in (1, 3, 17):
        parts = [rlk.logprob_from_logits(x[i:i + split], y[i:i + split], 0.7, 0.95)
                 for i in range(0, N, split)]
        for k in ref:
            if ref[k] is not None:
                assert torch.equal(ref[k], torch.cat([p_[k] for p_ in parts])), (k, split)
    perm = torch.from_numpy(np.random.default_rng(2).permutation(N))
    pr = rlk.logprob_from_logits(x[perm.to(DEV)].contiguous(), y[perm], 0.7, 0.95)
    for k in ref:
        if ref[k] is not None:
            assert torch.equal(ref[k][perm.to(DEV)], pr[k]), k


@pytest.mark.parametrize("p", [0.95, 1.0])
def test_bf16_row_as_last_and_middle_row_of_a_block(p):
    """The bf16 kernel runs one block per CU over rows b, b + G, b + 2G, ...
    (G = min(N, CUs)); a block's last row is finished by all of its waves,
    every other row by four while the rest stream. With N = 2G + 3 rows
    holding 7 distinct rows in turn, each distinct row is scored both as a
    block's last row and as a middle row (and alone, N = 1): every output must
    be bitwise the same in every position."""
    G = torch.cuda.get_device_properties(0).multi_processor_count
    N, K = 2 * G + 3, 7
    w = synth.workload("qwen")
    base = synth.logits_rows(w, range(K))
    yb = synth.peak_targets(w, range(K))
    idx = np.arange(N) % K
    x = bf16_to_device(base[idx])
    y = torch.as_tensor(yb[idx])
    print(f"  rlk_logprob_from_logits N={N} G={G} V={w.V} p={p}", flush=True)
    out = rlk.logprob_from_logits(x, y, 0.7, p)
    torch.cuda.synchronize()
    last = np.arange(N) + G >= N
    for k, v in out.items():
        if v is None:
            continue
        v = host(v)
        for c in range(K):
            pos = np.flatnonzero(idx == c)
            assert last[pos].any() and (~last[pos]).any()
            ref = v[pos[0]]
            for q in pos[1:]:
                assert v[q].tobytes() == ref.tobytes(), (k, c, q, v[q], ref)
    for c in range(K):
        one = rlk.logprob_from_logits(bf16_to_device(base[c:c + 1]), torch.as_tensor(yb[c:c + 1]),
                                      0.7, p)
        for k, v in one.items():
            if v is not None:
                assert host(v)[0].tobytes() == host(out[k])[c].tobytes(), (k, c)
    o = OL.logprob_from_logits(OL.widen_bf16(base), yb, OL.f32(0.7), OL.f32(p))
    check({k: (None if v is None else host(v)[:K]) for k, v in out.items()}, o, **BF16_TOL)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 2, 3, 7, 9, 17])
@pytest.mark.parametrize("T,p", [(1.0, 1.0), (0.7, 0.5), (0.3, 0.95)])
def test_tiny_vocabularies(dtype, V, T, p):
    """V below one 16-byte vector and just past it: a one-token vocabulary
    (lp = 0, H = 0), ties across the whole row, a dominant token."""
    r = np.random.default_rng(V)
    rows = [r.normal(0, 2.0, V), np.full(V, 1.5), np.where(np.arange(V) == V - 1, 9.0, -1.0)]
    arr = np.stack(rows).astype(np.float32)
    if dtype == "bf16":
        arr = synth.bf16_bits_from_f32(arr).reshape(arr.shape)
    y = np.array([0, V // 2, V - 1], dtype=np.int64)
    z = widen(arr, dtype)
    o = OL.logprob_from_logits(z, y, OL.f32(T), OL.f32(p))
    g = run(arr, dtype, y, T, p)
    check(g, o, **(F32_TOL if dtype == "f32" else BF16_TOL))
    if V == 1:   # (the entropy is a difference of fp64 terms: zero to rounding)
        assert np.all(g["lp_full"] == 0) and np.all(g["lp_trunc"] == 0)
        assert np.all(np.abs(g["entropy_full"]) <= 1e-12) and np.all(g["nucleus_size"] == 1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_rows(dtype):
    V = 151936 if dtype == "bf16" else 8192
    x = torch.empty(0, V, device=DEV, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    print(f"  rlk_logprob_from_logits N=0 V={V} {dtype}", flush=True)
    out = rlk.logprob_from_logits(x, torch.empty(0, dtype=torch.int64), 0.7, 0.95)
    torch.cuda.synchronize()
    assert all(v is None or v.numel() == 0 for v in out.values())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_maximum_vocabulary(dtype):
    """V = 2^24, the largest vocabulary the boundary accepts: a Gaussian row
    and, in bf16, a constant row (one value held 2^24 times wraps its 16-bit
    counter, so the row is handed to the generic kernel), in fp32 a row with
    a dominant token."""
    V = 1 << 24
    r = np.random.default_rng(77)
    second = (np.full(V, -1.25) if dtype == "bf16"
              else np.where(np.arange(V) == 12345, 20.0, r.normal(0, 1.0, V)))
    rows = np.stack([r.normal(0, 2.5, V), second]).astype(np.float32)
    arr = synth.bf16_bits_from_f32(rows).reshape(rows.shape) if dtype == "bf16" else rows
    y = np.array([7, 12345], dtype=np.int64)
    print(f"  oracle on 2 x {V} ({dtype})", flush=True)
    o = OL.logprob_from_logits(widen(arr, dtype), y, OL.f32(0.7), OL.f32(0.95))
    g = run(arr, dtype, y, 0.7, 0.95)
    check(g, o, **(F32_TOL if dtype == "f32" else BF16_TOL))
