"""Index arithmetic of the bf16 pattern-counting kernel, checked on the host
against the definitions it stands for (every 16-bit pattern, every thread of
both finisher sizes). The kernel keeps one 32-bit counter pair per magnitude
in the window [0x2000, 0x6000) (|z| in [2^-63, 2^64)), stored rotated: index
= magnitude & 0x3fff; the positive pattern counts in the low 16 bits, the
negative one in the high 16 bits."""
import numpy as np

PAT = np.arange(0x10000, dtype=np.uint32)


def in_window(pat):
    mag = pat & 0x7FFF
    return (mag >= 0x2000) & (mag < 0x6000)


def test_window_test_by_16_bit_add():
    # the streaming loop adds 0x2000 to each 16-bit half (no carry between
    # halves) and tests bit 14 of the sum
    t = (PAT + 0x2000) & 0xFFFF
    assert np.array_equal((t & 0x4000) != 0, in_window(PAT))
    # ... for both halves of a word at once
    rng = np.random.default_rng(0)
    words = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    lo, hi = words & 0xFFFF, words >> 16
    packed = ((lo + 0x2000) & 0xFFFF) | (((hi + 0x2000) & 0xFFFF) << 16)
    both = (packed & 0x40004000) == 0x40004000
    assert np.array_equal(both, in_window(lo) & in_window(hi))


def test_counter_offset_and_increment():
    words = (PAT[:, None] | (PAT[None, ::1021] << 16)).ravel().astype(np.uint32)
    lo, hi = words & 0xFFFF, words >> 16
    # byte offset of a pattern's counter word: 4 * (magnitude & 0x3fff)
    assert np.array_equal((words & 0x3FFF) << 2, 4 * ((lo & 0x7FFF) & 0x3FFF))
    assert np.array_equal(((words >> 16) & 0x3FFF) << 2, 4 * ((hi & 0x7FFF) & 0x3FFF))
    # increment: each half's sign spread over the half (arithmetic shift of
    # the 16-bit value by 15), plus 1: 1 for a positive pattern, 0x10000
    # for a negative one
    sg_lo = ((lo.astype(np.int32) << 16) >> 31).astype(np.uint32) & 0xFFFF
    sg_hi = ((hi.astype(np.int32) << 16) >> 31).astype(np.uint32) & 0xFFFF
    sg = sg_lo | (sg_hi << 16)
    want_lo = np.where(lo & 0x8000, 0x10000, 1)
    want_hi = np.where(hi & 0x8000, 0x10000, 1)
    assert np.array_equal((sg & 0xFFFF) + 1, want_lo)
    assert np.array_equal((sg >> 16) + 1, want_hi)


def wmag(i):
    """Magnitude held by counter index i (the rotation's inverse)."""
    return np.where(i < 0x2000, i + 0x4000, i)


def test_group_magnitude_per_finisher_thread():
    # the sweep's group q = ft + k*FT covers counters 4q .. 4q+3, whose first
    # magnitude the kernel forms as 4 ft + 4 k FT, plus 0x4000 when
    # 4 k FT < 0x2000; and the four magnitudes of a group are consecutive
    for FT in (256, 1024):
        assert 0x2000 % (4 * FT) == 0
        ft = np.arange(FT)
        for k in range(16384 // 4 // FT):
            base = 4 * ft + 4 * k * FT + (0x4000 if 4 * k * FT < 0x2000 else 0)
            assert np.array_equal(base, wmag(4 * (ft + k * FT)))
            for j in range(4):
                assert np.array_equal(base + j, wmag(4 * (ft + k * FT) + j))


def test_occupied_range_groups_cover_every_counter_once():
    # the Z pass and the clearing visit groups g0 + 4 g, g < ng, with
    # g0 = wmin & ~3 and ng = ((wmax | 3) - g0 + 1) / 4; each is one
    # contiguous 16-byte read at counter index (g0 + 4 g) & 0x3fff
    rng = np.random.default_rng(1)
    for _ in range(200):
        wmin, wmax = np.sort(rng.integers(0x2000, 0x6000, 2))
        g0 = wmin & ~3
        ng = ((wmax | 3) - g0 + 1) >> 2
        mags = (g0 + 4 * np.arange(ng))[:, None] + np.arange(4)[None, :]
        idx = (g0 + 4 * np.arange(ng)) & 0x3FFF
        assert np.array_equal(mags.ravel(), np.arange(g0, (wmax | 3) + 1))
        assert np.array_equal(wmag(idx[:, None] + np.arange(4)[None, :]), mags)
        assert (idx % 4 == 0).all() and idx.max() + 3 < 0x4000
