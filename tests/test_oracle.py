"""Pins of the CPU oracle to things other than itself (CPU only).

* the plain definition -- block-masked attention over [K; K_mem] -- written
  with no roll and no reshape, against the shift/partition pipeline;
* torch's scaled-dot-product attention in float64 (a library routine) for the
  cases that reduce to full or masked attention;
* closed forms worked by hand on tiny inputs;
* invariants of the method (shift period, roll equivariance, permutation
  equivariance inside windows, memory order, convexity);
* explicit loops for the mean pooling.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def sdpa(q, k, v, mask=None, scale=None):
    """torch float64 scaled-dot-product attention (library routine)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=m, scale=scale).numpy()


# ---------------------------------------------------------------- hand-worked
def test_hand_example_shift_direction():
    """1x4 grid, windows of 2, shift 1 along x, D = 1, scale 1.

    With the grid rolled by -1 the windows are {1, 2} and {3, 0}, so token 0
    attends keys 0 and 3, token 2 attends keys 1 and 2.
    """
    q = np.array([1.0, 0.0, 2.0, -1.0])
    k = np.array([0.0, 1.0, -1.0, 2.0])
    v = np.array([10.0, 20.0, 30.0, 40.0])
    e = math.exp
    expect = [
        (10 + e(2) * 40) / (1 + e(2)),                 # keys 0, 3 (logits 0, 2)
        25.0,                                          # q = 0: plain mean of 20, 30
        (e(2) * 20 + e(-2) * 30) / (e(2) + e(-2)),      # keys 1, 2 (logits 2, -2)
        (10 + e(-2) * 40) / (1 + e(-2)),               # keys 0, 3 (logits 0, -2)
    ]
    sh = lambda a: a.reshape(1, 1, 4, 1)
    out = O.window_attention(sh(q), sh(k), sh(v), (1, 4), (1, 2), (0, 1), scale=1.0)
    np.testing.assert_allclose(out.reshape(-1), expect, rtol=1e-14)
    assert list(O.window_id((1, 4), (1, 2), (0, 1))) == [1, 0, 0, 1]


def test_hand_example_memory():
    """Same 1x4 grid with a (1,2) mean pool of the unshifted grid.

    Memory keys: mean(k0,k1) = 0.5, mean(k2,k3) = 0.5; values 15 and 35.
    Token 0 (q = 1) sees keys 0, 3 and both memory tokens under one softmax.
    """
    q = np.array([1.0, 0.0, 2.0, -1.0])
    k = np.array([0.0, 1.0, -1.0, 2.0])
    v = np.array([10.0, 20.0, 30.0, 40.0])
    sh = lambda a: a.reshape(1, 1, 4, 1)
    km = O.pool_mean(sh(k), (1, 4), (1, 2))
    vm = O.pool_mean(sh(v), (1, 4), (1, 2))
    np.testing.assert_allclose(km.reshape(-1), [0.5, 0.5], rtol=0, atol=0)
    np.testing.assert_allclose(vm.reshape(-1), [15.0, 35.0], rtol=0, atol=0)
    e = math.exp
    o0 = (10 + e(2) * 40 + e(0.5) * 15 + e(0.5) * 35) / (1 + e(2) + 2 * e(0.5))
    o1 = (20 + 30 + 15 + 35) / 4.0
    o2 = (e(2) * 20 + e(-2) * 30 + e(1) * 15 + e(1) * 35) / (e(2) + e(-2) + 2 * e(1))
    o3 = (10 + e(-2) * 40 + e(-0.5) * (15 + 35)) / (1 + e(-2) + 2 * e(-0.5))
    out = O.window_attention(sh(q), sh(k), sh(v), (1, 4), (1, 2), (0, 1), km, vm,
                             scale=1.0)
    np.testing.assert_allclose(out.reshape(-1), [o0, o1, o2, o3], rtol=1e-14)
    # token-count corrected memory: each memory logit gains ln(2)
    oc = O.window_attention(sh(q), sh(k), sh(v), (1, 4), (1, 2), (0, 1), km, vm,
                            scale=1.0, mem_logit_bias=math.log(2.0))
    o1c = (20 + 30 + 2 * 15 + 2 * 35) / 6.0
    assert abs(oc.reshape(-1)[1] - o1c) < 1e-13


# ------------------------------------------------- pipeline vs plain definition
GEOMS = [
    ((4, 6), (2, 3)), ((6, 4), (3, 2)), ((8, 8), (4, 4)), ((5, 10), (5, 5)),
    ((3, 4, 6), (3, 2, 3)), ((4, 6, 5), (2, 3, 5)), ((2, 3, 4), (1, 1, 2)),
]


@pytest.mark.parametrize("grid,window", GEOMS)
@pytest.mark.parametrize("with_mem", [False, True])
def test_pipeline_equals_masked_definition(grid, window, with_mem):
    D = 8
    n = int(np.prod(grid))
    q, k, v = (rnd((2, 2, n, D), s) for s in (1, 2, 3))
    pool = tuple(w for w in window) if with_mem else None
    shifts = list(itertools.product(*[range(-1, w + 2) for w in window]))
    rng = np.random.default_rng(7)
    picks = [shifts[i] for i in rng.choice(len(shifts), size=min(12, len(shifts)),
                                            replace=False)]
    for s in picks:
        km = vm = None
        if pool is not None:
            km, vm = O.pool_mean(k, grid, pool), O.pool_mean(v, grid, pool)
        a = O.window_attention(q, k, v, grid, window, s, km, vm)
        b = O.masked_attention_bruteforce(q, k, v, grid, window, s, km, vm)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_masked_definition_equals_library_sdpa():
    """The brute-force definition equals torch SDPA with the same mask."""
    grid, window, shift = (3, 4, 6), (3, 2, 3), (1, 1, 2)
    n, D, G = 72, 8, 0
    q, k, v = (rnd((1, 2, n, D), s) for s in (4, 5, 6))
    km, vm = O.pool_mean(k, grid, (1, 2, 3)), O.pool_mean(v, grid, (1, 2, 3))
    G = km.shape[2]
    ref = O.masked_attention_bruteforce(q, k, v, grid, window, shift, km, vm)
    # mask from explicit coordinates (x fastest), not from window_id
    T, Hg, Wg = grid
    coords = [(t, y, x) for t in range(T) for y in range(Hg) for x in range(Wg)]

    def win(c):
        return tuple(((c[i] - shift[i]) % grid[i]) // window[i] for i in range(3))

    mask = np.array([[win(a) == win(b) for b in coords] + [True] * G for a in coords])
    kc = np.concatenate([k, km], axis=2)
    vc = np.concatenate([v, vm], axis=2)
    np.testing.assert_allclose(ref, sdpa(q, kc, vc, mask), rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------- invariants
def test_I1_window_equals_grid_is_full_attention():
    grid = (6, 10)
    q, k, v = (rnd((2, 3, 60, 16), s) for s in (10, 11, 12))
    out = O.window_attention(q, k, v, grid, grid, (0, 0))
    np.testing.assert_allclose(out, sdpa(q, k, v), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.full_attention(q, k, v), sdpa(q, k, v),
                               rtol=1e-12, atol=1e-12)
    rows = [0, 7, 59]
    np.testing.assert_allclose(O.full_attention(q, k, v, rows=rows),
                               sdpa(q, k, v)[:, :, rows], rtol=1e-12, atol=1e-12)


def test_I1_with_memory_is_full_attention_over_concat():
    grid, pool = (4, 6), (2, 3)
    q, k, v = (rnd((1, 2, 24, 8), s) for s in (13, 14, 15))
    km, vm = O.pool_mean(k, grid, pool), O.pool_mean(v, grid, pool)
    out = O.window_attention(q, k, v, grid, grid, (0, 0), km, vm)
    ref = sdpa(q, np.concatenate([k, km], 2), np.concatenate([v, vm], 2))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_scale_argument_matches_library():
    grid = (4, 4)
    q, k, v = (rnd((1, 1, 16, 8), s) for s in (16, 17, 18))
    out = O.window_attention(q, k, v, grid, grid, (0, 0), scale=0.3)
    np.testing.assert_allclose(out, sdpa(q, k, v, scale=0.3), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("grid,window", GEOMS[:5])
def test_I2_shift_period(grid, window):
    n = int(np.prod(grid))
    q, k, v = (rnd((1, 1, n, 4), s) for s in (20, 21, 22))
    s = tuple(1 for _ in window)
    a = O.window_attention(q, k, v, grid, window, s)
    s2 = tuple(si + 2 * w for si, w in zip(s, window))
    s3 = tuple(si - w for si, w in zip(s, window))
    np.testing.assert_allclose(a, O.window_attention(q, k, v, grid, window, s2), atol=0)
    np.testing.assert_allclose(a, O.window_attention(q, k, v, grid, window, s3), atol=0)
    z = tuple(0 for _ in window)
    np.testing.assert_allclose(O.window_attention(q, k, v, grid, window, window),
                               O.window_attention(q, k, v, grid, window, z), atol=0)


def test_I3_roll_and_partition_are_invertible():
    from oracle.basa_oracle import _partition, _roll_grid, _unpartition
    grid3, win3, s3 = (4, 6, 10), (2, 3, 5), (1, -2, 7)
    x = rnd((2, 240, 3), 30)
    y = _roll_grid(_roll_grid(x, grid3, s3, -1), grid3, s3, +1)
    np.testing.assert_array_equal(x, y)
    np.testing.assert_array_equal(_unpartition(_partition(x, grid3, win3), grid3, win3), x)
    idx = O.window_token_index((4, 6, 10), (2, 3, 5), s3)
    assert sorted(idx.reshape(-1).tolist()) == list(range(240))


def test_I4_permutation_equivariance_inside_windows():
    grid, window, shift = (6, 9), (3, 3), (1, 2)
    n = 54
    q, k, v = (rnd((1, 2, n, 6), s) for s in (31, 32, 33))
    wid = O.window_id(grid, window, shift)
    rng = np.random.default_rng(34)
    perm = np.arange(n)
    for w in np.unique(wid):
        members = np.nonzero(wid == w)[0]
        perm[members] = rng.permutation(members)
    a = O.window_attention(q, k, v, grid, window, shift)
    b = O.window_attention(q[:, :, perm], k[:, :, perm], v[:, :, perm], grid, window, shift)
    np.testing.assert_allclose(b, a[:, :, perm], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("with_mem", [False, True])
def test_I5_roll_equivariance(with_mem):
    grid, window, pool = (4, 6, 8), (2, 3, 4), (2, 3, 2)
    q, k, v = (rnd((1, 1, 192, 4), s) for s in (40, 41, 42))
    s = (1, 2, 1)
    delta = (2, 3, 4) if with_mem else (1, 1, 3)   # multiples of the pool with memory

    def roll(x, d):
        g = x.reshape((1, 1) + grid + (4,))
        return np.roll(g, d, axis=(2, 3, 4)).reshape(x.shape)

    def run(q, k, v, sh):
        km = vm = None
        if with_mem:
            km, vm = O.pool_mean(k, grid, pool), O.pool_mean(v, grid, pool)
        return O.window_attention(q, k, v, grid, window, sh, km, vm)

    a = roll(run(q, k, v, s), delta)
    b = run(roll(q, delta), roll(k, delta), roll(v, delta),
            tuple(si + di for si, di in zip(s, delta)))
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_I6_memory_order_invariance():
    grid, window, pool = (8, 8), (4, 4), (2, 4)
    q, k, v = (rnd((1, 2, 64, 8), s) for s in (50, 51, 52))
    km, vm = O.pool_mean(k, grid, pool), O.pool_mean(v, grid, pool)
    p = np.random.default_rng(53).permutation(km.shape[2])
    a = O.window_attention(q, k, v, grid, window, (2, 1), km, vm)
    b = O.window_attention(q, k, v, grid, window, (2, 1), km[:, :, p], vm[:, :, p])
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_I7_closed_forms():
    grid = (4, 6)
    q, k, v = (rnd((1, 2, 24, 8), s) for s in (60, 61, 62))
    # single-token windows, no memory: each token attends only itself
    np.testing.assert_allclose(O.window_attention(q, k, v, grid, (1, 1), (0, 0)), v,
                               rtol=1e-14, atol=1e-14)
    # constant V rows: output equals that row whatever the weights
    vc = np.broadcast_to(rnd((1, 2, 1, 8), 63), v.shape).copy()
    km, vm = O.pool_mean(k, grid, (2, 2)), O.pool_mean(vc, grid, (2, 2))
    np.testing.assert_allclose(O.window_attention(q, k, vc, grid, (2, 3), (1, 2), km, vm),
                               vc, rtol=1e-13, atol=1e-13)
    # pool = whole grid: one memory token, the mean of all tokens
    np.testing.assert_allclose(O.pool_mean(k, grid, grid)[:, :, 0], k.mean(axis=2),
                               rtol=1e-14)
    # pool = window, shift 0: memory token j is the mean of window j
    idx = O.window_token_index(grid, (2, 3), (0, 0))
    km = O.pool_mean(k, grid, (2, 3))
    for j in range(idx.shape[0]):
        np.testing.assert_allclose(km[:, :, j], k[:, :, idx[j]].mean(axis=2), rtol=1e-13)


def test_I8_convexity():
    grid, window, shift, pool = (6, 6), (3, 3), (1, 2), (3, 2)
    q, k, v = (rnd((1, 1, 36, 5), s) for s in (70, 71, 72))
    q = q * 4.0
    km, vm = O.pool_mean(k, grid, pool), O.pool_mean(v, grid, pool)
    out = O.window_attention(q, k, v, grid, window, shift, km, vm)
    wid = O.window_id(grid, window, shift)
    for i in range(36):
        vals = np.concatenate([v[0, 0, wid == wid[i]], vm[0, 0]], axis=0)
        assert np.all(out[0, 0, i] <= vals.max(axis=0) + 1e-12)
        assert np.all(out[0, 0, i] >= vals.min(axis=0) - 1e-12)


def test_I9_shift_schedule_matches_workload_text():
    with open(os.path.join(GOLDEN, "shift_schedules.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        for b, want in enumerate(c["shifts"]):
            assert list(O.shift_for_block(b, c["schedule"], c["window"])) == want, c["name"]
    # 3D four-phase: binary counting over the axes (t, y, x)
    got = [O.shift_for_block(b, O.SCHED_FOUR_PHASE, (7, 10, 13)) for b in range(8)]
    assert got == [(0, 0, 0), (3, 0, 0), (0, 5, 0), (3, 5, 0), (0, 0, 6), (3, 0, 6),
                   (0, 5, 6), (3, 5, 6)]


def test_I10_pool_equals_loops():
    grid, pool = (4, 6, 8), (2, 3, 2)
    x = rnd((2, 1, 192, 3), 80)
    got = O.pool_mean(x, grid, pool)
    T, Hg, Wg = grid
    G = 0
    for gt in range(T // 2):
        for gy in range(Hg // 3):
            for gx in range(Wg // 2):
                acc = np.zeros((2, 1, 3))
                for a in range(2):
                    for b in range(3):
                        for c in range(2):
                            t, y, xx = gt * 2 + a, gy * 3 + b, gx * 2 + c
                            acc += x[:, :, (t * Hg + y) * Wg + xx]
                np.testing.assert_allclose(got[:, :, G], acc / 12.0, rtol=1e-14)
                G += 1
    assert G == O.mem_tokens(grid, pool) == got.shape[2]


def test_window_token_index_matches_definition():
    grid, window, shift = (3, 4, 6), (3, 2, 3), (2, -1, 4)
    idx = O.window_token_index(grid, window, shift)
    wid = O.window_id(grid, window, shift)
    for j in range(idx.shape[0]):
        assert np.all(wid[idx[j]] == j)


def test_work_model():
    # dense over window flops is the n/m ratio of the complexity argument
    n, m, G, D = 16384, 256, 256, 128
    assert O.dense_flops(1, 24, n, D) / O.window_flops(1, 24, n, m, 0, D) == n / m
    assert O.theoretical_speedup(n, m) == 64.0
    assert O.theoretical_speedup(n, m, G) == 32.0


def test_head_sampling_matches_full():
    grid, window, shift, pool = (8, 12), (4, 4), (2, 3), (4, 4)
    q, k, v = (rnd((1, 2, 96, 8), s) for s in (90, 91, 92))
    km, vm = O.pool_mean(k, grid, pool), O.pool_mean(v, grid, pool)
    full = O.window_attention(q, k, v, grid, window, shift, km, vm)
    idx, out = O.window_attention_head(q[0, 1], k[0, 1], v[0, 1], grid, window, shift,
                                       km[0, 1], vm[0, 1], windows=[1, 4])
    np.testing.assert_allclose(out, full[0, 1][idx], rtol=1e-13, atol=1e-13)


def test_errors():
    q = np.zeros((1, 1, 24, 4))
    with pytest.raises(ValueError):
        O.window_attention(q, q, q, (4, 6), (3, 3), (0, 0))
    with pytest.raises(ValueError):
        O.pool_mean(q, (4, 6), (3, 3))
    with pytest.raises(ValueError):
        O.shift_for_block(-1, 1, (2, 2))


# ------------------------------------------------------------ property tests
@st.composite
def geometry(draw):
    ndim = draw(st.sampled_from([2, 3]))
    window = tuple(draw(st.integers(1, 5)) for _ in range(ndim))
    mult = tuple(draw(st.integers(1, 3)) for _ in range(ndim))
    grid = tuple(w * k for w, k in zip(window, mult))
    if int(np.prod(grid)) > 300:
        grid = window
    shift = tuple(draw(st.integers(-7, 9)) for _ in range(ndim))
    pool = None
    if draw(st.booleans()):
        pool = tuple(draw(st.sampled_from([d for d in range(1, g + 1) if g % d == 0]))
                     for g in grid)
    D = draw(st.sampled_from([4, 8, 16]))
    B = draw(st.integers(1, 2))
    H = draw(st.integers(1, 2))
    seed = draw(st.integers(0, 10_000))
    return ndim, grid, window, shift, pool, D, B, H, seed


@settings(max_examples=60, deadline=None)
@given(geometry())
def test_property_pipeline_equals_definition(g):
    ndim, grid, window, shift, pool, D, B, H, seed = g
    n = int(np.prod(grid))
    q, k, v = (rnd((B, H, n, D), seed + i) for i in range(3))
    km = vm = None
    if pool is not None:
        km, vm = O.pool_mean(k, grid, pool), O.pool_mean(v, grid, pool)
    a = O.window_attention(q, k, v, grid, window, shift, km, vm)
    b = O.masked_attention_bruteforce(q, k, v, grid, window, shift, km, vm)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)
