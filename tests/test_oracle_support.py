"""Pins of oracle.support (retained-set scoring) against library routines,
closed forms, the independently pinned nucleus oracle and invariants."""
import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import logprob, support


def _row(seed, V=200, scale=2.0):
    r = np.random.default_rng(seed)
    return r.normal(0, scale, V)


def test_full_support_is_the_library_softmax():
    z = _row(1)
    T = 0.7
    ids = np.arange(z.size)
    for y in (0, 17, 199):
        lp, h, fl = support.row(z, y, T, ids)
        assert fl == 0
        assert lp == pytest.approx(scipy.special.log_softmax(z / T)[y], rel=1e-13, abs=1e-13)
        assert h == pytest.approx(scipy.stats.entropy(scipy.special.softmax(z / T)), rel=1e-12)


def test_subset_is_the_library_softmax_of_the_subset():
    z = _row(2)
    T = 1.3
    ids = np.array([3, 8, 9, 50, 120, 199])
    lp, h, fl = support.row(z, 50, T, ids)
    ref = scipy.special.log_softmax(z[ids] / T)
    assert fl == 0
    assert lp == pytest.approx(ref[3], rel=1e-13)
    assert h == pytest.approx(scipy.stats.entropy(np.exp(ref)), rel=1e-12)


def test_closed_forms():
    z = _row(3)
    lp, h, fl = support.row(z, 7, 0.9, [7])               # one token: certain
    assert (lp, h, fl) == (0.0, 0.0, 0)
    zz = np.full(64, 1.25)                                  # k equal logits: uniform
    lp, h, fl = support.row(zz, 5, 0.5, np.arange(0, 64, 3))
    k = len(range(0, 64, 3))
    assert fl == support.FLAG_OUTSIDE and lp == -np.inf     # 5 is not a multiple of 3
    assert h == pytest.approx(np.log(k), rel=1e-14)
    lp, h, fl = support.row(zz, 6, 0.5, np.arange(0, 64, 3))
    assert lp == pytest.approx(-np.log(k), rel=1e-14) and fl == 0


def test_nucleus_support_matches_the_truncated_outputs():
    """S = the top-p nucleus: the truncated outputs of the pinned nucleus oracle."""
    for seed, T, p in ((4, 0.7, 0.95), (5, 1.0, 0.5), (6, 1.8, 0.99)):
        z = _row(seed, V=500)
        y = int(np.argsort(z)[-3])
        r = logprob.row(z, y, T, p)
        lp, h, fl = support.row(z, y, T, np.flatnonzero(r.keep), check_p=p)
        assert lp == pytest.approx(r.lp_trunc, rel=1e-13)
        assert h == pytest.approx(r.h_trunc, rel=1e-12)
        assert fl & support.FLAG_MISMATCH == 0


def test_mismatch_against_the_nucleus():
    z = _row(7, V=300)
    T, p = 0.7, 0.9
    keep = logprob.nucleus(z, T, p)[0]
    ids = np.flatnonzero(keep)
    y = int(ids[0])
    assert support.row(z, y, T, ids[:-1], check_p=p)[2] & support.FLAG_MISMATCH
    extra = np.sort(np.append(ids, np.flatnonzero(~keep)[0]))
    assert support.row(z, y, T, extra, check_p=p)[2] & support.FLAG_MISMATCH
    assert support.row(z, y, T, ids, check_p=p)[2] & support.FLAG_MISMATCH == 0
    assert support.row(z, y, T, np.arange(z.size), check_p=1.0)[2] == 0


def test_boundary_row_accepts_either_nucleus():
    # the top group (two equal values) holds all but about e^-50 of the mass,
    # within 1e-6 of p: the next group could come in, so both sets are valid
    z = np.array([0.0, 0.0, -50.0, -60.0])
    keep, tau, m_gt, m_ge, alts = logprob.nucleus(z, 1.0, 0.999999999)
    assert alts, "a boundary row"
    for k in [keep] + alts:
        fl = support.row(z, 0, 1.0, np.flatnonzero(k), check_p=0.999999999)[2]
        assert fl & support.FLAG_BOUNDARY and not fl & support.FLAG_MISMATCH


def test_invariants():
    z = _row(8)
    ids = np.array([1, 4, 9, 16, 25, 36, 49, 64, 81, 100])
    lp, h, _ = support.row(z, 36, 0.8, ids)
    lp2, h2, _ = support.row(z + 123.0, 36, 0.8, ids)      # shift invariance
    assert lp2 == pytest.approx(lp, rel=1e-11) and h2 == pytest.approx(h, rel=1e-11)
    lp3, h3, _ = support.row(z / 0.8, 36, 1.0, ids)         # T folds into the logits
    assert lp3 == pytest.approx(lp, rel=1e-12) and h3 == pytest.approx(h, rel=1e-12)
    # adding a token with tiny mass barely moves the outputs, lowers lp
    z2 = z.copy()
    z2[150] = z[ids].max() - 60.0
    lp4, h4, _ = support.row(z2, 36, 0.8, np.sort(np.append(ids, 150)))
    assert lp4 <= lp and abs(lp4 - lp) <= 1e-15 and abs(h4 - h) <= 1e-15


@pytest.mark.parametrize("ids,flag", [([], support.FLAG_BAD_SUPPORT),
                                      ([3, 3], support.FLAG_BAD_SUPPORT),
                                      ([5, 2], support.FLAG_BAD_SUPPORT),
                                      ([0, 200], support.FLAG_BAD_SUPPORT),
                                      ([-1, 4], support.FLAG_BAD_SUPPORT)])
def test_invalid_supports(ids, flag):
    lp, h, fl = support.row(_row(9), 0, 1.0, ids)
    assert fl & flag and np.isnan(lp) and np.isnan(h)


def test_nonfinite_and_bad_target():
    z = _row(10)
    z[4] = np.nan
    lp, h, fl = support.row(z, 0, 1.0, [0, 4, 9])
    assert fl & support.FLAG_NONFINITE and np.isnan(lp) and np.isnan(h)
    lp, h, fl = support.row(z, 0, 1.0, [0, 5, 9])            # the NaN is outside S
    assert fl == 0 and np.isfinite(lp)
    lp, h, fl = support.row(_row(11), 500, 1.0, [0, 5])
    assert fl == support.FLAG_BAD_TARGET and np.isnan(lp) and np.isfinite(h)


def test_batch_and_csr():
    r = np.random.default_rng(12)
    z = r.normal(0, 2, (5, 40))
    masks = r.random((5, 40)) < 0.3
    masks[:, 0] = True
    offsets, ids = support.csr_from_masks(masks)
    assert offsets[0] == 0 and offsets[-1] == ids.size and ids.dtype == np.int32
    y = np.zeros(5, dtype=np.int64)
    out = support.logprob_from_support(z, y, 0.7, offsets, ids)
    for n in range(5):
        lp, h, fl = support.row(z[n], 0, 0.7, np.flatnonzero(masks[n]))
        assert (out.lp[n], out.h[n], out.flags[n], out.size[n]) == (lp, h, fl, masks[n].sum())


def test_top_k_check():
    """The check against a top-k/top-p nucleus: the top-k nucleus itself
    passes, the plain top-p nucleus (a different set here) is a mismatch."""
    rng = np.random.default_rng(51)
    z = rng.normal(0, 1.5, 300)
    T, p, k = 0.8, 0.95, 10
    keep_k, *_ = logprob.nucleus(z, T, p, top_k=k)
    keep_p, *_ = logprob.nucleus(z, T, p)
    assert keep_k.sum() <= k < keep_p.sum()
    y = int(np.argmax(z))
    _, _, f = support.row(z, y, T, np.flatnonzero(keep_k), check_p=p, check_k=k)
    assert not f & support.FLAG_MISMATCH
    _, _, f = support.row(z, y, T, np.flatnonzero(keep_p), check_p=p, check_k=k)
    assert f & support.FLAG_MISMATCH
    _, _, f = support.row(z, y, T, np.flatnonzero(keep_p), check_p=p)
    assert not f & support.FLAG_MISMATCH
