"""Pins of oracle.philox (published known-answer vectors) and of the sampler
definition oracle.sampling.sample_row (law of the draws, support, limits)."""
import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import logprob, philox, sampling


# Known-answer vectors of Philox-4x32 with 10 rounds as published with the
# generator's reference implementation (Random123, Salmon et al., SC 2011):
# (counter, key) -> output.
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    got = philox.philox4x32([np.array([c]) for c in ctr], [np.array([k]) for k in key])
    assert tuple(int(g[0]) for g in got) == want


def test_row_uniforms_layout_and_range():
    u = philox.row_uniforms(seed=0x0123456789abcdef, offset=7, row_key=(5 << 32) | 9, n=10)
    w = philox.philox4x32([np.array([1]), np.array([9]), np.array([5]), np.array([7])],
                          [np.array([0x89abcdef]), np.array([0x01234567])])
    assert u[4] == (int(w[0][0]) + 0.5) * 2.0 ** -32 and u[7] == (int(w[3][0]) + 0.5) * 2.0 ** -32
    big = philox.row_uniforms(1, 0, 0, 1 << 16)
    assert np.all((big > 0) & (big < 1))
    # uniform on (0, 1): Kolmogorov-Smirnov at a fixed seed
    assert scipy.stats.kstest(big, "uniform").pvalue > 1e-3
    assert not np.array_equal(philox.row_uniforms(1, 1, 0, 64), big[:64])   # offset matters
    assert not np.array_equal(philox.row_uniforms(1, 0, 1, 64), big[:64])   # row key matters


def test_sample_row_law():
    """Over many offsets the draws follow softmax(z / T) on the nucleus."""
    z = np.array([2.0, 1.5, 1.0, 0.2, -1.0, -3.0])
    T, p = 0.7, 0.9
    keep, *_ = logprob.nucleus(z, T, p)
    q = np.zeros(z.size)
    q[keep] = scipy.special.softmax(z[keep] / T)
    draws = 20000
    counts = np.bincount([sampling.sample_row(z, T, p, 42, off, 3) for off in range(draws)],
                         minlength=z.size)
    assert np.all(counts[~keep] == 0)
    sd = np.sqrt(draws * q * (1 - q)) + 1e-9
    assert np.all(np.abs(counts - draws * q) <= 5 * sd)


def test_sample_row_limits():
    r = np.random.default_rng(0)
    z = r.normal(0, 2, 500)
    # a tiny top-p keeps the argmax only (all of a tied top group); -inf
    # tokens are never drawn; rows with a NaN or no finite logit give -1
    assert sampling.sample_row(z, 1.0, 1e-6, 1, 0, 0) == int(np.argmax(z))
    zt = z.copy()
    zt[[10, 20]] = z.max() + 1.0                  # two tied top values, both kept
    picks = {sampling.sample_row(zt, 1.0, 1e-6, 1, off, 0) for off in range(64)}
    assert picks <= {10, 20} and len(picks) == 2
    zn = z.copy()
    zn[3] = np.nan
    assert sampling.sample_row(zn, 1.0, 0.9, 1, 0, 0) == -1
    zi = np.full(8, -np.inf)
    assert sampling.sample_row(zi, 1.0, 0.9, 1, 0, 0) == -1
    zm = z.copy()
    zm[::2] = -np.inf                              # -inf tokens are never drawn
    assert all(sampling.sample_row(zm, 1.0, 1.0, 2, off, 0) % 2 == 1 for off in range(200))


def test_sample_row_law_with_top_k():
    """With top-k the draws follow the tempered softmax renormalised over the
    top-k/top-p set, and never leave it."""
    from oracle import logprob as L
    z = np.array([2.0, 1.6, 1.5, 1.5, 0.3, -0.2, -1.0, 0.9])
    T, p, k = 0.8, 0.97, 4
    keep, *_ = L.nucleus(z, T, p, top_k=k)
    assert keep.sum() == 4
    q = np.zeros(z.size)
    q[keep] = np.exp(z[keep] / T) / np.exp(z[keep] / T).sum()
    draws = 20000
    counts = np.zeros(z.size)
    for off in range(draws):
        counts[sampling.sample_row(z, T, p, 7, off, 0, top_k=k)] += 1
    assert counts[~keep].sum() == 0
    sd = np.sqrt(draws * q * (1 - q)) + 1e-9
    assert np.all(np.abs(counts - draws * q) <= 5 * sd)
