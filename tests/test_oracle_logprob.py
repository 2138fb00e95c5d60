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
