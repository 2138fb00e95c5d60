"""Pins for the logprob/entropy/top-p oracle: closed forms, library routines,
50-digit arithmetic, brute-force nucleus enumeration and invariants.

None of these re-types the oracle's own formula: each checks it against
something the mathematics fixes independently.
"""
import itertools
import math

import mpmath
import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import logprob as L
from oracle import sampling

TEMPS = [0.2, 0.7, 1.0, 1.8]          # the temperatures the pages' suite covers
PS = [1e-6, 0.5, 0.95, 1.0]


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("V", [1, 2, 7, 8192])
@pytest.mark.parametrize("T", TEMPS)
@pytest.mark.parametrize("p", PS)
def test_uniform_row(V, T, p):
    z = np.full(V, 1.25)
    r = L.row(z, V // 2, T, p)
    assert r.size == V                      # all tokens tied: the whole row is kept
    assert r.lp_full == pytest.approx(-math.log(V), abs=1e-12)
    assert r.h_full == pytest.approx(math.log(V), abs=1e-12)
    assert r.lp_trunc == pytest.approx(-math.log(V), abs=1e-12)
    assert r.h_trunc == pytest.approx(math.log(V), abs=1e-12)
    assert r.flags == 0


@pytest.mark.parametrize("T", TEMPS)
def test_two_token_logistic(T):
    a, b = 0.3, -1.1
    x = (a - b) / T
    q = 1.0 / (1.0 + math.exp(-x))          # P(token 0), logistic
    r0 = L.row(np.array([a, b]), 0, T, 1.0)
    r1 = L.row(np.array([a, b]), 1, T, 1.0)
    assert r0.lp_full == pytest.approx(math.log(q), rel=1e-13)
    assert r1.lp_full == pytest.approx(math.log(1 - q), rel=1e-13)
    hb = -q * math.log(q) - (1 - q) * math.log(1 - q)
    assert r0.h_full == pytest.approx(hb, rel=1e-12)
    # p below q keeps only token 0; p just above q keeps both
    r = L.row(np.array([a, b]), 0, T, q * 0.999)
    assert r.size == 1 and r.lp_trunc == 0.0 and r.h_trunc == 0.0
    r = L.row(np.array([a, b]), 0, T, min(1.0, q * 1.001))
    assert r.size == 2


def test_one_hot_dominant():
    V = 64
    z = np.zeros(V)
    z[5] = 100.0
    r = L.row(z, 5, 1.0, 0.95)
    assert abs(r.lp_full) < 1e-38            # -log(1 + 63 e^-100)
    assert r.h_full < 1e-38 * 200
    assert r.size == 1 and r.lp_trunc == 0.0 and r.h_trunc == 0.0
    r = L.row(z, 6, 1.0, 0.95)               # any other target is outside the nucleus
    assert r.lp_trunc == -math.inf and r.flags & L.FLAG_OUTSIDE
    assert r.lp_full == pytest.approx(-100.0, abs=1e-9)


# ---------------------------------------------------------- library routines

@pytest.mark.parametrize("T", TEMPS)
def test_full_stats_match_scipy(T):
    rng = np.random.default_rng(7)
    for _ in range(20):
        V = int(rng.integers(2, 3000))
        z = rng.normal(0, 3, V)
        y = int(rng.integers(0, V))
        r = L.row(z, y, T, 1.0)
        ls = scipy.special.log_softmax(z / T)
        assert r.lp_full == pytest.approx(ls[y], rel=1e-12, abs=1e-12)
        assert r.h_full == pytest.approx(scipy.stats.entropy(np.exp(ls)), rel=1e-10, abs=1e-12)
        # p = 1 reduces to the full softmax
        assert r.size == V
        assert r.lp_trunc == pytest.approx(r.lp_full, rel=1e-13, abs=1e-13)
        assert r.h_trunc == pytest.approx(r.h_full, rel=1e-13, abs=1e-13)


def test_mpmath_50_digits():
    mpmath.mp.dps = 50
    rng = np.random.default_rng(11)
    for _ in range(10):
        V = int(rng.integers(2, 9))
        z = rng.normal(0, 2, V)
        T = float(rng.choice(TEMPS))
        p = float(rng.uniform(0.3, 0.99))
        y = int(np.argmax(z))               # the argmax is always in the nucleus
        r = L.row(z, y, T, p)
        w = [mpmath.exp(mpmath.mpf(float(v)) / T) for v in z]
        Zm = mpmath.fsum(w)
        assert r.lp_full == pytest.approx(float(mpmath.log(w[y] / Zm)), rel=1e-13, abs=1e-14)
        Hm = -mpmath.fsum(wi / Zm * mpmath.log(wi / Zm) for wi in w)
        assert r.h_full == pytest.approx(float(Hm), rel=1e-12, abs=1e-14)
        ws = [w[i] for i in range(V) if r.keep[i]]
        Zs = mpmath.fsum(ws)
        assert r.lp_trunc == pytest.approx(float(mpmath.log(w[y] / Zs)), rel=1e-13, abs=1e-14)
        Hs = -mpmath.fsum(wi / Zs * mpmath.log(wi / Zs) for wi in ws)
        assert r.h_trunc == pytest.approx(float(Hs), rel=1e-12, abs=1e-14)


# ------------------------------------------------------ brute-force nucleus

def _min_card(prob, p):
    """Smallest number of tokens whose probability mass reaches p (enumeration)."""
    V = len(prob)
    for k in range(1, V + 1):
        for sub in itertools.combinations(range(V), k):
            if sum(prob[i] for i in sub) >= p:
                return k
    return V


@pytest.mark.parametrize("ties", [False, True])
def test_nucleus_bruteforce(ties):
    rng = np.random.default_rng(3 + ties)
    for _ in range(150):
        V = int(rng.integers(1, 11))
        z = rng.integers(-3, 3, V).astype(float) if ties else rng.normal(0, 2, V)
        T = float(rng.choice(TEMPS))
        p = float(rng.uniform(0.05, 0.999))
        prob = scipy.special.softmax(z / T)
        k = _min_card(prob, p)
        keep, tau, m_gt, m_ge, alts = L.nucleus(z, T, p)
        if alts:                              # too close to the boundary to decide
            continue
        kth = np.sort(z)[::-1][k - 1]         # value of the k-th most probable token
        np.testing.assert_array_equal(keep, z >= kth)
        if not ties:
            assert keep.sum() == k


# ---------------------------------------------------------------- invariants

def _rows(seed, n=30):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        V = int(rng.integers(2, 400))
        z = rng.normal(0, float(rng.choice([0.5, 2.0, 5.0])), V)
        if rng.random() < 0.5:               # bf16-like coarse values: many ties
            z = np.round(z * 8) / 8
        yield z, float(rng.choice(TEMPS)), float(rng.choice([0.1, 0.5, 0.9, 0.95, 0.999]))


def test_nucleus_invariants():
    for z, T, p in _rows(5):
        keep, tau, m_gt, m_ge, alts = L.nucleus(z, T, p)
        prob = scipy.special.softmax(z / T)
        assert prob[keep].sum() >= p - 1e-12                       # mass reaches p
        lowest = keep & (z == z[keep].min())
        assert prob[keep & ~lowest].sum() < p + 1e-12              # minimal: drop the lowest group
        assert np.all(keep[z >= z[keep].min()])                    # value-closed
        assert keep[np.argmax(z)]                                  # argmax group always kept
        assert np.array_equal(L.nucleus(z, T, 1.0)[0], np.ones(z.size, bool))
        tiny = L.nucleus(z, T, 1e-9)[0]
        np.testing.assert_array_equal(tiny, z == z.max())          # p -> 0+: argmax group


def test_truncated_invariants():
    for z, T, p in _rows(9, n=15):
        r0 = L.row(z, int(np.argmax(z)), T, p)
        S = np.flatnonzero(r0.keep)
        lps = np.array([L.row(z, int(y), T, p).lp_trunc for y in S])
        assert np.exp(lps).sum() == pytest.approx(1.0, rel=1e-12)  # renormalised
        # lp_trunc - lp_full = -log P(S), the same for every target in S
        shift = lps - np.array([L.row(z, int(y), T, p).lp_full for y in S])
        prob = scipy.special.softmax(z / T)
        np.testing.assert_allclose(shift, -math.log(prob[S].sum()), rtol=1e-11, atol=1e-12)
        assert r0.h_trunc <= math.log(S.size) + 1e-12
        assert r0.lp_trunc >= r0.lp_full - 1e-15


def test_tied_nucleus_entropy_is_log_size():
    z = np.array([3.0, 3.0, 3.0, 3.0, 3.0, -2.0, -2.5, -4.0])
    r = L.row(z, 0, 0.7, 0.9)
    assert r.size == 5
    assert r.h_trunc == pytest.approx(math.log(5), abs=1e-14)
    assert r.lp_trunc == pytest.approx(-math.log(5), abs=1e-14)


def test_exact_equality_excludes_group():
    # two tokens of mass exactly 1/2 each: M_>(second) = 1/2 = p, so the
    # second group is excluded and only the first is kept
    z = np.array([1.0, 0.0])
    T = 1.0 / math.log(3.0)                  # masses 3/4 and 1/4
    keep, tau, m_gt, m_ge, _ = L.nucleus(z, T, 0.75)
    assert m_ge == pytest.approx(0.75, abs=1e-15)
    assert keep.tolist() in ([True, False], [True, True])   # exact tie with p is a boundary case
    keep, *_ = L.nucleus(z, T, 0.7)
    assert keep.tolist() == [True, False]
    keep, *_ = L.nucleus(z, T, 0.8)
    assert keep.tolist() == [True, True]


# ------------------------------------------------------------ edge cases

def test_neg_inf_entries():
    z = np.array([2.0, -np.inf, 1.0, -np.inf])
    r = L.row(z, 0, 1.0, 1.0)
    assert r.size == 2                                     # p = 1 keeps finite tokens only
    assert r.lp_full == pytest.approx(-math.log1p(math.exp(-1.0)), rel=1e-14)
    r = L.row(z, 1, 1.0, 0.5)
    assert r.lp_full == -math.inf and r.lp_trunc == -math.inf and r.flags & L.FLAG_OUTSIDE


def test_nonfinite_and_bad_target():
    r = L.row(np.array([1.0, np.nan, 0.0]), 0, 1.0, 0.9)
    assert r.flags & L.FLAG_NONFINITE and math.isnan(r.lp_full)
    r = L.row(np.array([1.0, np.inf, 0.0]), 0, 1.0, 0.9)
    assert r.flags & L.FLAG_NONFINITE
    r = L.row(np.array([-np.inf, -np.inf]), 0, 1.0, 0.9)
    assert r.flags & L.FLAG_NONFINITE
    r = L.row(np.array([1.0, 0.0]), 2, 1.0, 0.9)
    assert r.flags & L.FLAG_BAD_TARGET and math.isnan(r.lp_full)
    assert not math.isnan(r.h_trunc)


def test_boundary_flag_and_alternative():
    # masses 0.5 / 0.3 / 0.2 (T = 1): with p = 0.8 exactly the inclusive mass
    # of the second group equals p, a boundary row with an alternative set
    z = np.log(np.array([0.5, 0.3, 0.2]))
    r = L.row(z, 0, 1.0, 0.8)
    assert r.flags & L.FLAG_BOUNDARY
    sizes = sorted([r.size] + [int(a.sum()) for a in r.alt_keeps])
    assert sizes in ([2, 3], [1, 2])


# ------------------------------------------------------------ sampler

def test_gumbel_target_in_nucleus_and_distribution():
    rng = np.random.default_rng(0)
    z = np.array([2.0, 1.5, 1.0, 0.2, -1.0, -3.0])
    T, p = 0.7, 0.9
    keep, *_ = L.nucleus(z, T, p)
    q = np.zeros(z.size)
    q[keep] = scipy.special.softmax(z[keep] / T)
    draws = 20000
    counts = np.zeros(z.size)
    for _ in range(draws):
        u = rng.random(z.size) * (1 - 2e-16) + 1e-16
        y = sampling.gumbel_max_target(z, T, p, u)
        assert keep[y]
        counts[y] += 1
    sd = np.sqrt(draws * q * (1 - q)) + 1e-9
    assert np.all(np.abs(counts - draws * q) <= 5 * sd)


# ------------------------------------------------- input widening (bf16 -> fp64)

def test_widen_bf16_all_patterns_match_torch():
    """Every one of the 65536 bf16 bit patterns widens to the value torch's own
    bf16 -> fp32 conversion gives (fp32 -> fp64 is exact), NaNs to NaNs."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = L.widen_bf16(bits)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    theirs = t.numpy().astype(np.float64)
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 * 127                       # exponent all ones, mantissa != 0
    np.testing.assert_array_equal(ours[~nan], theirs[~nan])
    # the sign of zero survives
    assert math.copysign(1.0, ours[0x8000]) == -1.0 and math.copysign(1.0, ours[0]) == 1.0


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xBF80, -1.0), (0x4000, 2.0), (0x3F00, 0.5),
    (0x4049, 3.140625),                       # sign 0, exponent 128, mantissa 0x49
    (0x3F81, 1.0 + 2.0 ** -7),                # one unit of the 7-bit mantissa
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),  # the largest finite bf16
    (0x0080, 2.0 ** -126),                    # the smallest normal
    (0x0001, 2.0 ** -133),                    # the smallest subnormal
    (0x7F80, math.inf), (0xFF80, -math.inf),
])
def test_widen_bf16_known_values(bits, value):
    # the values follow from the format alone: 1 sign, 8 exponent (bias 127)
    # and 7 mantissa bits, subnormals at exponent 0
    assert L.widen_bf16(np.array([bits], dtype=np.uint16))[0] == value


# ------------------------------------------------------ the batch wrapper

def test_batch_per_row_parameters_match_single_rows():
    """Per-row T and p arrays reach each row: the batch equals the rows one by
    one, and a row with (T, p) = (1, 1) gives scipy's log-softmax."""
    rng = np.random.default_rng(21)
    N, V = 12, 300
    z = rng.normal(0, 2, (N, V))
    z[3] = np.round(z[3] * 4) / 4                      # a tie-heavy row
    y = rng.integers(0, V, N)
    Ts = rng.choice(TEMPS, N)
    ps = rng.choice([0.3, 0.9, 0.95, 1.0], N)
    Ts[5], ps[5] = 1.0, 1.0
    b = L.logprob_from_logits(z, y, Ts, ps)
    for n in range(N):
        r = L.row(z[n], int(y[n]), float(Ts[n]), float(ps[n]))
        for got, want in ((b.lp_full[n], r.lp_full), (b.h_full[n], r.h_full),
                          (b.lp_trunc[n], r.lp_trunc), (b.h_trunc[n], r.h_trunc),
                          (b.tau[n], r.tau)):
            assert got == want or (math.isnan(got) and math.isnan(want))
        assert b.size[n] == r.size and b.flags[n] == r.flags
    ls = scipy.special.log_softmax(z[5])
    assert b.lp_full[5] == pytest.approx(ls[y[5]], rel=1e-12, abs=1e-12)
    assert b.lp_trunc[5] == pytest.approx(ls[y[5]], rel=1e-12, abs=1e-12)
    # scalar parameters broadcast to every row
    s = L.logprob_from_logits(z, y, 0.7, 0.95)
    assert np.array_equal(s.size, [L.row(z[n], int(y[n]), 0.7, 0.95).size for n in range(N)])


def test_batch_boundary_alternatives_are_the_other_valid_sets():
    """A boundary row's alternative tuples hold the statistics of the other
    valid nucleus, checked against closed forms of an equal-logit group."""
    # masses (T = 1): a group of 2 equal tokens with 0.25 each, then 5 equal
    # tokens with 0.1 each. p = 0.5 exactly equals the top group's mass, so
    # keeping the top group (|S| = 2) and keeping everything (|S| = 7) are
    # both valid within the boundary tolerance.
    z = np.log(np.array([0.25, 0.25, 0.1, 0.1, 0.1, 0.1, 0.1]))
    y = np.array([0, 4])
    b = L.logprob_from_logits(np.stack([z, z]), y, 1.0, 0.5)
    for n in range(2):
        assert b.flags[n] & L.FLAG_BOUNDARY
        sets = {b.size[n]: (b.lp_trunc[n], b.h_trunc[n])}
        for alt in b.alts[n]:
            sets[alt[0]] = alt[1:]
        assert sorted(sets) == [2, 7]
        # |S| = 2: uniform over the top pair; token 4 is outside it
        lp2, h2 = sets[2]
        assert h2 == pytest.approx(math.log(2), abs=1e-14)
        assert (lp2 == pytest.approx(-math.log(2), abs=1e-14)) if n == 0 else lp2 == -math.inf
        # |S| = 7: the whole row, masses 0.25 x2 and 0.1 x5
        lp7, h7 = sets[7]
        assert lp7 == pytest.approx(math.log(0.25 if n == 0 else 0.1), abs=1e-14)
        assert h7 == pytest.approx(-(2 * 0.25 * math.log(0.25) + 5 * 0.1 * math.log(0.1)),
                                   abs=1e-14)
    # a row away from the boundary has no alternatives
    far = L.logprob_from_logits(z[None, :], y[:1], 1.0, 0.6)
    assert far.alts[0] == [] and not far.flags[0] & L.FLAG_BOUNDARY


# ------------------------------------------------------------------ top-k

def _kth_by_count(z, k):
    """v_k by counting: the largest row value v with #{z_i >= v} >= k."""
    vals = sorted(set(z.tolist()), reverse=True)
    for v in vals:
        if sum(1 for x in z if x >= v) >= k:
            return v
    return vals[-1]


@pytest.mark.parametrize("ties", [False, True])
def test_top_k_then_top_p_bruteforce(ties):
    """S = the smallest value-closed set inside the top-k set S_k (ties with the
    k-th value kept) whose mass, renormalised over S_k, reaches p: checked by
    enumerating subsets of S_k on tiny rows."""
    rng = np.random.default_rng(31 + ties)
    checked = 0
    for _ in range(200):
        V = int(rng.integers(1, 10))
        z = rng.integers(-3, 3, V).astype(float) if ties else rng.normal(0, 2, V)
        k = int(rng.integers(1, V + 2))
        T = float(rng.choice(TEMPS))
        p = float(rng.choice([rng.uniform(0.05, 0.999), 1.0]))
        vk = _kth_by_count(z, k)
        Sk = z >= vk
        keep, tau, _, _, alts = L.nucleus(z, T, p, top_k=k)
        assert np.all(keep <= Sk)                                  # inside the top-k set
        if p >= 1.0:
            np.testing.assert_array_equal(keep, Sk)
            continue
        if alts:
            continue
        idx = np.flatnonzero(Sk)
        prob = scipy.special.softmax(z[idx] / T)                   # renormalised over S_k
        kmin = _min_card(prob, p)
        kth = np.sort(z[idx])[::-1][kmin - 1]
        np.testing.assert_array_equal(keep, Sk & (z >= kth))
        checked += 1
    assert checked > 50


def test_top_k_closed_forms():
    rng = np.random.default_rng(41)
    z = rng.normal(0, 2, 50)
    y = int(np.argmax(z))
    r = L.row(z, y, 0.7, 1.0, top_k=1)                 # k = 1, distinct values: the argmax
    assert r.size == 1 and r.lp_trunc == 0.0 and r.h_trunc == 0.0 and r.tau == z.max()
    r = L.row(z, (y + 1) % 50, 0.7, 1.0, top_k=1)
    assert r.lp_trunc == -math.inf and r.flags & L.FLAG_OUTSIDE
    # k levels: k tokens at a, the rest at b < a; top-k = k keeps exactly the k
    for k in (1, 3, 7):
        zz = np.array([2.5] * k + [-1.0] * (20 - k))
        r = L.row(zz, 0, 0.9, 1.0, top_k=k)
        assert r.size == k and r.tau == 2.5
        assert r.lp_trunc == pytest.approx(-math.log(k), abs=1e-14)
        assert r.h_trunc == pytest.approx(math.log(k), abs=1e-14)
        # the full statistics stay those of the whole row
        full = scipy.special.log_softmax(zz / 0.9)
        assert r.lp_full == pytest.approx(full[0], rel=1e-13)
    # ties at the k-th value are all kept: 4 equal values, k = 2
    zz = np.array([3.0, 1.0, 1.0, 1.0, 1.0, -2.0])
    r = L.row(zz, 4, 1.0, 1.0, top_k=2)
    assert r.size == 5 and r.tau == 1.0
    # k at or above the finite count: no filtering
    zz = np.array([1.0, -np.inf, 0.5, 0.25])
    for k in (3, 4, 100):
        a, b = L.row(zz, 0, 0.8, 0.9, top_k=k), L.row(zz, 0, 0.8, 0.9)
        assert (a.size, a.lp_trunc, a.h_trunc) == (b.size, b.lp_trunc, b.h_trunc)
    # uniform row: every k keeps the whole tie group
    r = L.row(np.full(16, 0.5), 3, 0.7, 0.3, top_k=5)
    assert r.size == 16 and r.lp_trunc == pytest.approx(-math.log(16), abs=1e-14)


def test_top_k_invariants():
    """Renormalising over S_k only raises relative masses, so the top-k/top-p
    set lies inside both S_k and the plain top-p set; the full statistics do
    not depend on k; k = 0 is the plain rule."""
    for z, T, p in _rows(17, n=40):
        for k in (1, 2, 5, 17, 60):
            keep, tau, *_ = L.nucleus(z, T, p, top_k=k)
            keep0, *_ = L.nucleus(z, T, p)
            vk = L.top_k_floor(z, k)
            assert np.all(keep <= (z >= vk)) and np.all(keep <= keep0)
            assert keep[np.argmax(z)]
            assert np.all(keep[z >= z[keep].min()])             # value-closed
            a, b = L.row(z, 0, T, p, top_k=k), L.row(z, 0, T, p)
            assert a.lp_full == b.lp_full and a.h_full == b.h_full
        np.testing.assert_array_equal(L.nucleus(z, T, p, top_k=0)[0], L.nucleus(z, T, p)[0])


def test_top_k_per_row_batch():
    rng = np.random.default_rng(43)
    z = rng.normal(0, 2, (6, 40))
    y = rng.integers(0, 40, 6)
    ks = np.array([0, 1, 3, 40, 7, 2])
    b = L.logprob_from_logits(z, y, 0.7, 0.95, top_k=ks)
    for n in range(6):
        r = L.row(z[n], int(y[n]), 0.7, 0.95, top_k=int(ks[n]))
        assert b.size[n] == r.size and b.tau[n] == r.tau
        assert b.lp_trunc[n] == r.lp_trunc or (math.isnan(b.lp_trunc[n]) and math.isnan(r.lp_trunc))
