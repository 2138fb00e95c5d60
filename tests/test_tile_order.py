"""Tile order of the tile GEMM (tile_of_block in mfma_gemm.h), restated here
and checked on the host: it must be a bijection from workgroup index onto the
na x nb tile grid for every grid shape (each output tile computed exactly
once), and inside a full super-tile of 32 x 8 tiles the workgroups one XCD
receives (every 8th, dealt round-robin) must form an 8 x 4 block."""
import itertools

import pytest

SUP_A, SUP_B, SUB_A, SUB_B, XCDS = 32, 8, 8, 4, 8


def tile_of_block(na, nb, b):
    band, i = divmod(b, SUP_A * nb)
    ga = min(SUP_A, na - band * SUP_A)
    blk, j = divmod(i, ga * SUP_B)
    gb = min(SUP_B, nb - blk * SUP_B)
    if ga == SUP_A and gb == SUP_B:
        parts_a = SUP_A // SUB_A
        x, s = j % XCDS, j // XCDS
        a = (x % parts_a) * SUB_A + s % SUB_A
        c = (x // parts_a) * SUB_B + s // SUB_A
    else:
        a, c = j % ga, j // ga
    return band * SUP_A + a, blk * SUP_B + c


# grids of the workloads (Qwen3 head at 8192 and 16384 tokens, Llama head,
# the backward's dh and dW grids) and ragged ones around the super-tile size
GRIDS = [(594, 32), (594, 64), (501, 64), (430, 16), (128, 16), (82, 16), (1, 1), (7, 3),
         (31, 7), (32, 8), (33, 9), (64, 16), (65, 17), (40, 40), (3, 300), (300, 3)]


@pytest.mark.parametrize("na,nb", GRIDS)
def test_bijection(na, nb):
    seen = [tile_of_block(na, nb, b) for b in range(na * nb)]
    assert all(0 <= a < na and 0 <= c < nb for a, c in seen)
    assert len(set(seen)) == na * nb


def test_xcd_parts_of_a_full_super_tile():
    na, nb = 64, 16   # 2 x 2 full super-tiles
    for st in range(4):
        base = st * SUP_A * SUP_B
        for x in range(XCDS):
            tiles = [tile_of_block(na, nb, base + x + XCDS * s) for s in range(SUB_A * SUB_B)]
            rows = sorted({a for a, _ in tiles})
            cols = sorted({c for _, c in tiles})
            assert len(rows) == SUB_A and len(cols) == SUB_B
            assert rows == list(range(rows[0], rows[0] + SUB_A))
            assert cols == list(range(cols[0], cols[0] + SUB_B))
            assert set(tiles) == set(itertools.product(rows, cols))
