"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Bars: bf16 max abs <= 2e-2 and mean abs <= 2e-3; fp32 max abs <= 1e-5, both
against the float64 oracle on the exact input values.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import (assert_close, bhnd_to_bnhd, log, make_full_inputs, random_geometry,
                      random_qkv, to_gpu, to_np)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_window_attention_amd")


def _sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------- tiny fp32
@pytest.mark.parametrize("shift", [(4, 4), (0, 0), (-3, 9)])
def test_tiny_f32(shift):
    wl = W.TINY
    log(f"tiny fp32 shift={shift}")
    q, k, v = W.make_qkv(wl)
    out = S.window_attn(to_gpu(q, "f32"), to_gpu(k, "f32"), to_gpu(v, "f32"), wl.grid, wl.window,
                        shift, scale=1.0 / math.sqrt(64))
    _sync()
    ref = O.window_attention(q, k, v, wl.grid, wl.window, shift)
    assert_close(to_np(out), ref, "f32", f"tiny shift {shift}")


# ---------------------------------------------------- small multi-tile, ragged
SMALL = [
    # grid, window, pool, shift
    ((24, 40), (12, 20), (4, 8), (5, 13)),
    ((6, 10, 26), (3, 5, 13), (3, 5, 2), (1, 3, 7)),
    ((6, 10, 26), (3, 5, 13), (1, 5, 13), (-1, -2, 20)),
    ((16, 48), (16, 16), None, (8, 3)),
    ((7, 9), (7, 9), (7, 9), (0, 0)),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_geometries(case, D, dtype):
    grid, window, pool, shift = SMALL[case]
    n = int(np.prod(grid))
    B, H = 2, 3
    log(f"small case={case} D={D} dtype={dtype} grid={grid} window={window} pool={pool}")
    q, k, v = random_qkv((B, H, n, D), dtype, seed=100 + case)
    qg, kg, vg = (to_gpu(x, dtype) for x in (q, k, v))
    mem = None
    km = vm = None
    if pool is not None:
        mem = S.pool_kv(kg, vg, grid, pool)
        km, vm = O.pool_mean(k, grid, pool), O.pool_mean(v, grid, pool)
    out = S.window_attn(qg, kg, vg, grid, window, shift, mem=mem)
    _sync()
    ref = O.window_attention(q, k, v, grid, window, shift, km, vm)
    assert_close(to_np(out), ref, dtype, f"small {case} D{D} {dtype}")


@pytest.mark.parametrize("seed", range(24))
def test_random_geometries(seed):
    grid, window, shift, pool, D, dtype, layout, B, H, bias = random_geometry(1000 + seed)
    n = int(np.prod(grid))
    log(f"random geometry seed={seed} grid={grid} window={window} shift={shift} pool={pool} "
        f"D={D} {dtype} {layout} B={B} H={H} bias={bias:.3f}")
    q, k, v = random_qkv((B, H, n, D), dtype, seed=2000 + seed)
    km = vm = None
    if pool is not None:
        km, vm = O.pool_mean(k, grid, pool), O.pool_mean(v, grid, pool)
    ref = O.window_attention(q, k, v, grid, window, shift, km, vm, mem_logit_bias=bias)
    conv = bhnd_to_bnhd if layout == "bnhd" else (lambda x: x)
    qg, kg, vg = (to_gpu(conv(x), dtype) for x in (q, k, v))
    mem = S.pool_kv(kg, vg, grid, pool, layout=layout) if pool is not None else None
    out = S.window_attn(qg, kg, vg, grid, window, shift, mem=mem, mem_bias=bias, layout=layout)
    _sync()
    got = to_np(out)
    if layout == "bnhd":
        got = np.transpose(got, (0, 2, 1, 3))
    assert_close(got, ref, dtype, f"random geometry {seed}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bnhd_layout(dtype):
    grid, window, pool, shift = SMALL[0]
    n, B, H, D = int(np.prod(grid)), 2, 3, 128
    log(f"bnhd layout {dtype}")
    q, k, v = random_qkv((B, H, n, D), dtype, seed=7)
    ref = O.window_attention(q, k, v, grid, window, shift, O.pool_mean(k, grid, pool),
                             O.pool_mean(v, grid, pool))
    qg, kg, vg = (to_gpu(bhnd_to_bnhd(x), dtype) for x in (q, k, v))
    mem = S.pool_kv(kg, vg, grid, pool, layout="bnhd")
    out = S.window_attn(qg, kg, vg, grid, window, shift, mem=mem, layout="bnhd")
    _sync()
    got = np.transpose(to_np(out), (0, 2, 1, 3))
    assert_close(got, ref, dtype, f"bnhd {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_token_count_corrected_memory(dtype):
    grid, window, pool, shift = (16, 32), (8, 8), (4, 4), (3, 5)
    n, B, H, D = 512, 1, 2, 64
    log(f"memory logit bias {dtype}")
    q, k, v = random_qkv((B, H, n, D), dtype, seed=8)
    bias = math.log(16.0)
    qg, kg, vg = (to_gpu(x, dtype) for x in (q, k, v))
    mem = S.pool_kv(kg, vg, grid, pool)
    out = S.window_attn(qg, kg, vg, grid, window, shift, mem=mem, mem_bias=bias)
    _sync()
    ref = O.window_attention(q, k, v, grid, window, shift, O.pool_mean(k, grid, pool),
                             O.pool_mean(v, grid, pool), mem_logit_bias=bias)
    assert_close(to_np(out), ref, dtype, f"mem bias {dtype}")


# Persistent kernel (at least four key tiles per unit) with a memory logit
# bias: tiles of memory keys only take the bias as one offset of the row max
# and the exponent; a tile straddling the window/memory boundary or holding
# padding keys takes it per key.
BIAS_PERSISTENT = [
    # grid, window, pool: m = 256 with G = 256 (four memory-only tiles) and
    # G = 80 (one memory-only tile, then one with padding keys); m = 400
    # with G = 80 (a tile straddling window and memory keys, padding keys)
    ((64, 64), (16, 16), (4, 4)),
    ((64, 80), (16, 16), (8, 8)),
    ((40, 80), (20, 20), (5, 8)),
]


@pytest.mark.parametrize("case", range(len(BIAS_PERSISTENT)))
def test_memory_bias_persistent(case):
    grid, window, pool = BIAS_PERSISTENT[case]
    n, B, H, D = int(np.prod(grid)), 1, 3, 128
    shift = (window[0] // 2, 3)
    bias = math.log(float(np.prod(pool)))
    log(f"memory bias, persistent: grid={grid} window={window} pool={pool}")
    q, k, v = random_qkv((B, H, n, D), "bf16", seed=500 + case)
    qg, kg, vg = (to_gpu(x, "bf16") for x in (q, k, v))
    mem = S.pool_kv(kg, vg, grid, pool)
    out = S.window_attn(qg, kg, vg, grid, window, shift, mem=mem, mem_bias=bias)
    _sync()
    ref = O.window_attention(q, k, v, grid, window, shift, O.pool_mean(k, grid, pool),
                             O.pool_mean(v, grid, pool), mem_logit_bias=bias)
    assert_close(to_np(out), ref, "bf16", f"mem bias persistent case {case}")


# ------------------------------------------------------------------ pooling
# (grid, pool, head dim): a wave's 64 / (16-byte chunks per row) lane groups
# split each cell row of px tokens, px a multiple of the group count or not
# (a partial last step); video cells of several frames, image cells, one-row
# cells, head dims 64 and 128
POOL_SHAPES = [((6, 20, 24), (3, 5, 4), 128),   # bf16 1 token per group and row, f32 2
               ((32, 32), (8, 8), 128),         # bf16 2, f32 4
               ((32, 48), (16, 16), 64),        # bf16 2, f32 4
               ((12, 15), (3, 5), 128),         # px not a multiple of the groups
               ((16, 16), (1, 4), 128),         # one row per cell
               ((2, 8, 12), (2, 2, 6), 64)]     # two frames, px not a multiple


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
@pytest.mark.parametrize("shape", range(len(POOL_SHAPES)))
def test_pool_kv(dtype, layout, shape):
    grid, pool, D = POOL_SHAPES[shape]
    n, B, H = int(np.prod(grid)), 2, 2
    log(f"pool {dtype} {layout} grid={grid} pool={pool} D={D}")
    _, k, v = random_qkv((B, H, n, D), dtype, seed=9 + shape)
    conv = bhnd_to_bnhd if layout == "bnhd" else (lambda x: x)
    km, vm = S.pool_kv(to_gpu(conv(k), dtype), to_gpu(conv(v), dtype), grid, pool, layout=layout)
    _sync()
    for got, x in ((km, k), (vm, v)):
        ref = O.pool_mean(x, grid, pool)
        err = np.abs(to_np(got) - ref)
        # bf16: one rounding of the mean (half an ulp, relative 2^-9) plus fp32 sums
        tol = (np.abs(ref) * 2.0 ** -8 + 1e-6) if dtype == "bf16" else (np.abs(ref) * 1e-6 + 1e-6)
        assert np.all(err <= tol), float(err.max())


# ------------------------------------------------------------ full-size configs
@pytest.mark.parametrize("block", [0, 1])
def test_flux1024_full(block):
    wl = W.FLUX1024
    shift = S.shift_for_block(block, wl.schedule, wl.window)
    log(f"flux1024 block={block} shift={shift}")
    q, k, v = W.make_qkv(wl)
    qg, kg, vg = (to_gpu(x, "bf16") for x in (q, k, v))
    mem = S.pool_kv(kg, vg, wl.grid, wl.pool)
    out = S.window_attn(qg, kg, vg, wl.grid, wl.window, shift, mem=mem)
    _sync()
    ref = O.window_attention(q, k, v, wl.grid, wl.window, shift, O.pool_mean(k, wl.grid, wl.pool),
                             O.pool_mean(v, wl.grid, wl.pool))
    assert_close(to_np(out), ref, "bf16", f"flux1024 block {block}")


def _full_size_check(wl, shifts, heads_of, variant=0, with_mem=True):
    """Window attention at the workload's full size, once per shift: the
    output starts NaN-filled, every element of every head must be written,
    and for each shift the whole output of the heads ``heads_of(shift)``
    (seeded workload values) must match the oracle."""
    all_heads = sorted({h for sh in shifts for h in heads_of(sh)})
    gpu, exact = make_full_inputs(wl, all_heads, variant)
    qg, kg, vg = gpu
    use_mem = with_mem and wl.pool is not None
    mem = S.pool_kv(kg, vg, wl.grid, wl.pool) if use_mem else None
    mems = {}
    for shift in shifts:
        log(f"{wl.name} shift={shift} heads={heads_of(shift)}")
        out = torch.full_like(qg, float("nan"))
        S.window_attn(qg, kg, vg, wl.grid, wl.window, shift, mem=mem, out=out)
        _sync()
        assert not bool(torch.isnan(out).any()), f"unwritten output elements, shift {shift}"
        for h in heads_of(shift):
            q, k, v = (x[None, None] for x in exact[h])
            if h not in mems:
                mems[h] = ((O.pool_mean(k, wl.grid, wl.pool), O.pool_mean(v, wl.grid, wl.pool))
                           if use_mem else (None, None))
            km, vm = mems[h]
            ref = O.window_attention(q, k, v, wl.grid, wl.window, shift, km, vm)[0, 0]
            assert_close(to_np(out[0, h]), ref, "bf16", f"{wl.name} head {h} shift {shift}")


def _schedule_shifts(wl, blocks):
    return [S.shift_for_block(b, wl.schedule, wl.window) for b in blocks]


@pytest.mark.parametrize("wl", [W.FLUX2048_W16, W.FLUX2048_W32], ids=lambda w: w.name)
def test_flux2048_full(wl):
    # every head of the last phase of the four-phase schedule, and three
    # heads of each of the other three phases, checked whole
    shifts = _schedule_shifts(wl, range(4))
    last = shifts[3]
    _full_size_check(wl, shifts,
                     lambda sh: list(range(wl.heads)) if sh == last else [0, 13, 23])


NOMEM = [W.FLUX2048_W16.with_(name="flux2048_128x128_w16_nomem", pool=None),
         W.FLUX2048_W32.with_(name="flux2048_128x128_w32_nomem", pool=None)]


@pytest.mark.parametrize("wl", NOMEM, ids=lambda w: w.name)
def test_flux2048_no_memory_full(wl):
    # 4 (w16) and 16 (w32) key tiles per unit and several units per
    # workgroup: the persistent kernel's shortest units, whose successor's
    # tile loads start in their second iteration
    _full_size_check(wl, _schedule_shifts(wl, (1, 3)), lambda sh: [0, 23])


@pytest.mark.parametrize("wl", [W.WAN, W.WAN_G1638], ids=lambda w: w.name)
def test_wan_full(wl):
    # both phases of the alternating schedule, three whole heads each
    _full_size_check(wl, _schedule_shifts(wl, range(2)), lambda sh: [0, 21, 39])


def test_ultra_full():
    # all 256 windows of two heads at the last phase of the schedule
    wl = W.ULTRA
    _full_size_check(wl, _schedule_shifts(wl, (3,)), lambda sh: [5, 19])


# ------------------------------------------------------ launch configurations
# Shapes chosen to drive each path of the bf16 launcher: the persistent kernel
# with several units per workgroup (including the fewest tiles it takes, a
# ragged unit count per XCD, an odd tile count padded with a masked tile, the
# memory-bias masked phase, head dim 64, the BNHD layout with B > 1), and the
# per-unit kernel for units of fewer than four tiles and for windows whose
# tables do not fit next to the persistent kernel's buffers.
PATHS = [
    # name, B, H, D, grid, window, pool, shift, mem_bias, layout
    ("min tiles, ragged units", 2, 37, 128, (48, 80), (16, 16), None, (8, 3), 0.0, "bhnd"),
    ("odd tiles + bias phase", 1, 64, 128, (40, 40), (20, 20), (8, 8), (10, 7), math.log(64.0), "bhnd"),
    ("head dim 64", 1, 80, 64, (32, 64), (16, 16), (8, 8), (5, 11), 0.0, "bhnd"),
    ("bnhd, batch 2", 2, 80, 128, (32, 32), (16, 16), (8, 8), (8, 8), 0.0, "bnhd"),
    ("short units", 1, 8, 128, (64, 64), (8, 8), (8, 8), (4, 4), 0.0, "bhnd"),
    ("window of 4096", 1, 2, 128, (64, 64), (64, 64), (16, 16), (31, 40), 0.0, "bhnd"),
]


@pytest.mark.parametrize("case", range(len(PATHS)))
def test_launch_paths(case):
    name, B, H, D, grid, window, pool, shift, bias, layout = PATHS[case]
    n = int(np.prod(grid))
    log(f"path '{name}': B={B} H={H} D={D} grid={grid} window={window} pool={pool}")
    q, k, v = random_qkv((B, H, n, D), "bf16", seed=300 + case)
    km = vm = None
    if pool is not None:
        km, vm = O.pool_mean(k, grid, pool), O.pool_mean(v, grid, pool)
    ref = O.window_attention(q, k, v, grid, window, shift, km, vm, mem_logit_bias=bias)
    conv = bhnd_to_bnhd if layout == "bnhd" else (lambda x: x)
    qg, kg, vg = (to_gpu(conv(x), "bf16") for x in (q, k, v))
    mem = S.pool_kv(kg, vg, grid, pool, layout=layout) if pool is not None else None
    out = S.window_attn(qg, kg, vg, grid, window, shift, mem=mem, mem_bias=bias, layout=layout)
    _sync()
    got = to_np(out)
    if layout == "bnhd":
        got = got.transpose(0, 2, 1, 3)
    assert_close(got, ref, "bf16", f"path {name}")


def test_full_attn_many_units():
    B, H, n, D = 1, 48, 2048, 128     # 384 units: several per workgroup
    log("full attention, several units per workgroup")
    q, k, v = random_qkv((B, H, n, D), "bf16", seed=21)
    out = S.full_attn(to_gpu(q, "bf16"), to_gpu(k, "bf16"), to_gpu(v, "bf16"))
    _sync()
    rows = np.unique(np.linspace(0, n - 1, 96).astype(np.int64))
    heads = [0, 17, 31, 47]
    got = to_np(out)[:, heads][:, :, rows]
    ref = O.full_attention(q[:, heads], k[:, heads], v[:, heads], rows=rows)
    assert_close(got, ref, "bf16", "full many units")


def test_full_attn_flux2048_sampled():
    """The dense kernel at the shape the speedup is measured on (24 heads of
    16384 tokens, D = 128): sampled query rows of two seeded heads."""
    wl = W.FLUX2048_W16
    heads = [5, 18]
    log(f"dense {wl.name} heads {heads}")
    (qg, kg, vg), exact = make_full_inputs(wl, heads)
    out = torch.full_like(qg, float("nan"))
    S.full_attn(qg, kg, vg, out=out)
    _sync()
    assert not bool(torch.isnan(out).any()), "unwritten output elements"
    rows = np.unique(np.linspace(0, wl.n_tokens - 1, 80).astype(np.int64))
    for h in heads:
        q, k, v = exact[h]
        ref = O.full_attention(q[None, None], k[None, None], v[None, None], rows=rows)[0, 0]
        got = to_np(out[0, h][torch.from_numpy(rows).to(out.device)])
        assert_close(got, ref, "bf16", f"dense {wl.name} head {h}")


# ------------------------------------------------------------- dense kernel
@pytest.mark.parametrize("dtype,n,D", [("bf16", 4096, 128), ("bf16", 1000, 128),
                                       ("bf16", 777, 64), ("f32", 300, 64), ("f32", 520, 128)])
def test_full_attn(dtype, n, D):
    B, H = 1, 3
    log(f"full attention {dtype} n={n} D={D}")
    q, k, v = random_qkv((B, H, n, D), dtype, seed=n + D)
    out = S.full_attn(to_gpu(q, dtype), to_gpu(k, dtype), to_gpu(v, dtype))
    _sync()
    rows = np.unique(np.linspace(0, n - 1, min(n, 300)).astype(np.int64))
    ref = O.full_attention(q, k, v, rows=rows)
    assert_close(to_np(out)[:, :, rows], ref, dtype, f"full {dtype} n{n} D{D}")


DENSE = [
    # dtype, n_q, n_kv, D, layout: the persistent kernel (>= 4 key tiles) and
    # the per-unit kernel, ragged query and key counts, more queries than
    # keys, the window batches of the composition baseline (256 x 512)
    ("bf16", 256, 512, 128, "bhnd"),
    ("bf16", 910, 1456, 128, "bhnd"),
    ("bf16", 100, 1000, 64, "bnhd"),
    ("bf16", 1000, 64, 128, "bhnd"),
    ("bf16", 3000, 200, 128, "bnhd"),
    ("f32", 300, 77, 64, "bhnd"),
    ("f32", 64, 520, 128, "bnhd"),
]


@pytest.mark.parametrize("case", range(len(DENSE)))
def test_dense_attn_unequal_lengths(case):
    dtype, nq, nkv, D, layout = DENSE[case]
    B, H = 2, 3
    log(f"dense {dtype} n_q={nq} n_kv={nkv} D={D} {layout}")
    rng = np.random.default_rng(600 + case)
    q = rng.standard_normal((B, H, nq, D), dtype=np.float32)
    k = rng.standard_normal((B, H, nkv, D), dtype=np.float32)
    v = rng.standard_normal((B, H, nkv, D), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = (W.round_bf16(x) for x in (q, k, v))
    conv = bhnd_to_bnhd if layout == "bnhd" else (lambda x: x)
    qg, kg, vg = (to_gpu(conv(x), dtype) for x in (q, k, v))
    out = torch.full_like(qg, float("nan"))
    S.dense_attn(qg, kg, vg, out=out, layout=layout)
    _sync()
    got = to_np(out)
    if layout == "bnhd":
        got = got.transpose(0, 2, 1, 3)
    assert_close(got, O.full_attention(q, k, v), dtype, f"dense {nq}x{nkv} {dtype}")


def test_window_equal_grid_matches_full_kernel():
    grid = (32, 32)
    log("window = grid vs dense kernel")
    q, k, v = random_qkv((1, 2, 1024, 128), "bf16", seed=11)
    qg, kg, vg = (to_gpu(x, "bf16") for x in (q, k, v))
    a = S.window_attn(qg, kg, vg, grid, grid, (0, 0))
    b = S.full_attn(qg, kg, vg)
    _sync()
    assert torch.equal(a, b)
    assert_close(to_np(a), O.full_attention(q, k, v), "bf16", "window=grid")


# ------------------------------------------------------- sentinels and guards
def test_output_fully_written_and_guards_intact():
    grid, window, pool, shift = SMALL[1]
    n, B, H, D = int(np.prod(grid)), 2, 3, 128
    log("NaN sentinel + guard canaries")
    q, k, v = random_qkv((B, H, n, D), "bf16", seed=12)
    qg, kg, vg = (to_gpu(x, "bf16") for x in (q, k, v))
    mem = S.pool_kv(kg, vg, grid, pool)
    numel = B * H * n * D
    pad = 4096
    buf = torch.full((numel + 2 * pad,), float("nan"), dtype=torch.bfloat16, device=qg.device)
    buf[:pad] = 7.0
    buf[-pad:] = -7.0
    out = buf[pad:pad + numel].view(B, H, n, D)
    S.window_attn(qg, kg, vg, grid, window, shift, mem=mem, out=out)
    _sync()
    assert bool(torch.isfinite(out).all())
    assert bool((buf[:pad] == 7.0).all()) and bool((buf[-pad:] == -7.0).all())


def test_deterministic_and_shift_period():
    wl = W.FLUX1024
    log("determinism and shift period")
    q, k, v = random_qkv((1, 4, wl.n_tokens, 128), "bf16", seed=13)
    qg, kg, vg = (to_gpu(x, "bf16") for x in (q, k, v))
    mem = S.pool_kv(kg, vg, wl.grid, wl.pool)
    a = S.window_attn(qg, kg, vg, wl.grid, wl.window, (8, 8), mem=mem)
    b = S.window_attn(qg, kg, vg, wl.grid, wl.window, (8, 8), mem=mem)
    c = S.window_attn(qg, kg, vg, wl.grid, wl.window, (8 + 16, 8 - 32), mem=mem)
    z0 = S.window_attn(qg, kg, vg, wl.grid, wl.window, (0, 0), mem=mem)
    zw = S.window_attn(qg, kg, vg, wl.grid, wl.window, (16, 16), mem=mem)
    _sync()
    assert torch.equal(a, b)
    assert torch.equal(a, c)
    assert torch.equal(z0, zw)
    assert not torch.equal(a, z0)


def test_concurrent_streams():
    """Calls on two streams at once (default priority) give the results of the
    same calls made one after the other: the library keeps no state shared
    between calls."""
    grid, window, pool = (64, 64), (16, 16), (8, 8)
    n, B, H, D = 4096, 1, 8, 128
    log("two streams")
    ins = []
    for seed in (900, 901):
        q, k, v = random_qkv((B, H, n, D), "bf16", seed=seed)
        ins.append(tuple(to_gpu(x, "bf16") for x in (q, k, v)))
    shifts = [(8, 8), (0, 8)]
    ref = []
    for (qg, kg, vg), sh in zip(ins, shifts):
        mem = S.pool_kv(kg, vg, grid, pool)
        ref.append(S.window_attn(qg, kg, vg, grid, window, sh, mem=mem))
    _sync()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(r) for r in ref]
    for rep in range(3):
        for o in outs:
            o.zero_()
        _sync()
        for st, (qg, kg, vg), sh, o in zip(streams, ins, shifts, outs):
            with torch.cuda.stream(st):
                mem = S.pool_kv(kg, vg, grid, pool)
                S.window_attn(qg, kg, vg, grid, window, sh, mem=mem, out=o)
        _sync()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"repetition {rep}"


def test_binding_errors_before_launch():
    x = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(S.BasaError):
        S.window_attn(x, x, x.clone(), (8, 8), (3, 8), (0, 0))
    with pytest.raises(S.BasaError):
        S.window_attn(x, x, x, (8, 8), (4, 4), (0, 0), out=x)    # out aliases q


def test_empty_batch():
    # zero-sized batch: every call succeeds through the C ABI and returns empty outputs
    log("empty batch")
    dev = torch.device("cuda:0")
    q, k, v = (torch.empty((0, 3, 64, 128), dtype=torch.bfloat16, device=dev) for _ in range(3))
    mem = S.pool_kv(k, v, (8, 8), (4, 4))
    assert tuple(mem[0].shape) == (0, 3, 4, 128)
    out = S.window_attn(q, k, v, (8, 8), (4, 4), (2, 2), mem=mem)
    assert tuple(out.shape) == (0, 3, 64, 128)
    assert tuple(S.full_attn(q, k, v).shape) == (0, 3, 64, 128)
    order = torch.arange(64, dtype=torch.int32, device=dev)
    assert tuple(S.curve_attn(q, k, v, order, 16, 3).shape) == (0, 3, 64, 128)
    _sync()
