"""Pins of the Hilbert-tile oracle (oracle/basa_curve.py) and the library's
host-side Hilbert order."""
import json
import math
import os

import numpy as np
import pytest

import oracle as O


@pytest.mark.parametrize("side", [1, 2, 4, 8, 32])
def test_hilbert_curve_properties(side):
    pts = O.hilbert_curve_xy(side)
    n = side * side
    assert len(set(pts)) == n and all(0 <= x < side and 0 <= y < side for x, y in pts)
    assert pts[0] == (0, 0) and pts[-1] == (side - 1, 0)
    for (x0, y0), (x1, y1) in zip(pts, pts[1:]):          # unit steps
        assert abs(x0 - x1) + abs(y0 - y1) == 1
    for k in range(1, int(math.log2(side)) + 1):           # aligned 4^k runs fill squares
        run = 4 ** k
        for start in range(0, n, run):
            xs = [p[0] for p in pts[start:start + run]]
            ys = [p[1] for p in pts[start:start + run]]
            assert max(xs) - min(xs) == 2 ** k - 1 and max(ys) - min(ys) == 2 ** k - 1
            assert min(xs) % 2 ** k == 0 and min(ys) % 2 ** k == 0


def test_hilbert_side_two_by_definition():
    # the curve of side 2 visits lower-left, upper-left, upper-right, lower-right
    assert O.hilbert_curve_xy(2) == [(0, 0), (0, 1), (1, 1), (1, 0)]


@pytest.mark.parametrize("side", [2, 4, 16, 64, 128])
def test_library_hilbert_order_matches_oracle(side):
    S = pytest.importorskip("sparse_window_attention_amd")
    assert np.array_equal(S.hilbert_order(side), O.hilbert_order(side))


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "center_region.json")


def _golden_regions():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _check_region(idx, case):
    idx = [int(x) for x in idx]
    Hg, Wg = case["grid"]
    ch, cw = case["size"]
    assert len(idx) == ch * cw
    assert divmod(idx[0], Wg) == tuple(case["first"])
    if "tokens" in case:
        assert idx == case["tokens"]
    else:
        assert idx[:cw] == case["first_row"] and idx[-1] == case["last"]


@pytest.mark.parametrize("case", range(7))
def test_oracle_center_region_hand_worked(case):
    c = _golden_regions()[case]
    _check_region(O.center_region(c["grid"], c["size"]), c)


@pytest.mark.parametrize("case", range(7))
def test_library_center_region_hand_worked(case):
    S = pytest.importorskip("sparse_window_attention_amd")
    c = _golden_regions()[case]
    _check_region(S.center_region_tokens(c["grid"], c["size"]), c)


@pytest.mark.parametrize("grid,size", [((9, 9), (3, 3)), ((9, 10), (4, 3)), ((2, 7), (1, 6)),
                                       ((16, 16), (16, 1)), ((33, 20), (8, 8))])
def test_oracle_center_region_is_centred_block(grid, size):
    # a whole size[0] x size[1] block of the grid in raster order, with as
    # many rows (columns) before it as after it, or one fewer
    idx = O.center_region(grid, size)
    ys, xs = np.divmod(idx, grid[1])
    rows, cols = sorted(set(ys.tolist())), sorted(set(xs.tolist()))
    assert rows == list(range(rows[0], rows[0] + size[0]))
    assert cols == list(range(cols[0], cols[0] + size[1]))
    assert list(idx) == sorted(idx) and len(idx) == size[0] * size[1]
    for before, n, s in ((rows[0], grid[0], size[0]), (cols[0], grid[1], size[1])):
        after = n - s - before
        assert after - before in (0, 1)


@pytest.mark.parametrize("tile,slide,mem", [(16, 0, False), (16, 5, True), (64, 40, True),
                                            (4, 1, False)])
def test_curve_attention_equals_masked_definition(tile, slide, mem):
    side, D = 8, 8
    n = side * side
    rng = np.random.default_rng(tile + slide)
    q, k, v = (rng.standard_normal((2, 2, n, D)) for _ in range(3))
    order = O.hilbert_order(side)
    km = vm = None
    if mem:
        reg = O.center_region((side, side), (2, 2))
        km, vm = k[:, :, reg], v[:, :, reg]
    a = O.curve_attention(q, k, v, order, tile, slide, km, vm)
    b = O.curve_attention_bruteforce(q, k, v, order, tile, slide, km, vm)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_raster_order_is_window_attention_on_a_row():
    # with the raster order, tiles are windows of a 1 x n grid shifted by slide
    n, D, tile, slide = 48, 8, 12, 7
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 2, n, D)) for _ in range(3))
    a = O.curve_attention(q, k, v, np.arange(n), tile, slide)
    b = O.window_attention(q, k, v, (1, n), (1, tile), (0, slide))
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
