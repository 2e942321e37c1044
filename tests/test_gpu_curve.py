"""GPU parity of attention in tiles of a token order (Hilbert curve, random
permutations, the raster order) and of the row gather, through the C ABI,
against the CPU oracle.  Bars as for window attention: bf16 max abs <= 2e-2
and mean abs <= 2e-3, fp32 max abs <= 1e-5."""
import numpy as np
import pytest

import oracle as O
from gpu_util import assert_close, bhnd_to_bnhd, log, random_qkv, to_gpu, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_window_attention_amd")


def _order(o):
    return torch.from_numpy(np.asarray(o, dtype=np.int32)).cuda()


CASES = [
    # side, tile, slide, central region (None = no memory)
    (32, 64, 0, None),
    (32, 64, 17, (4, 4)),
    (32, 128, 515, (2, 6)),
    (64, 256, 128, (8, 8)),     # window + memory spans five 64-key tiles
    (16, 16, 3, (3, 3)),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_hilbert_tiles(case, dtype):
    side, tile, slide, region = CASES[case]
    n, B, H, D = side * side, 1, 2, 128
    log(f"hilbert case={case} {dtype} side={side} tile={tile} slide={slide} region={region}")
    q, k, v = random_qkv((B, H, n, D), dtype, seed=300 + case)
    qg, kg, vg = (to_gpu(x, dtype) for x in (q, k, v))
    order = O.hilbert_order(side)
    mem = km = vm = None
    if region is not None:
        # the library's region goes to the GPU; the oracle's is the reference
        mem = S.gather_kv(kg, vg, _order(S.center_region_tokens((side, side), region)))
        reg = O.center_region((side, side), region)
        km, vm = k[:, :, reg], v[:, :, reg]
    out = S.curve_attn(qg, kg, vg, _order(S.hilbert_order(side)), tile, slide, mem=mem)
    torch.cuda.synchronize()
    ref = O.curve_attention(q, k, v, order, tile, slide, km, vm)
    assert_close(to_np(out), ref, dtype, f"hilbert {case} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
def test_random_order_ragged(dtype, layout):
    # a random permutation; tile 96 and 40 memory keys leave ragged key tiles
    n, tile, slide, B, H, D = 960, 96, 301, 2, 2, 64
    log(f"random order {dtype} {layout}")
    rng = np.random.default_rng(5)
    order = rng.permutation(n)
    idx = rng.choice(n, 40, replace=False)
    q, k, v = random_qkv((B, H, n, D), dtype, seed=9)
    ref = O.curve_attention(q, k, v, order, tile, slide, k[:, :, idx], v[:, :, idx],
                            mem_logit_bias=0.7)
    conv = (lambda x: x) if layout == "bhnd" else bhnd_to_bnhd
    qg, kg, vg = (to_gpu(conv(x), dtype) for x in (q, k, v))
    mem = S.gather_kv(kg, vg, _order(idx), layout=layout)
    out = S.curve_attn(qg, kg, vg, _order(order), tile, slide, mem=mem, mem_bias=0.7,
                       layout=layout)
    torch.cuda.synchronize()
    got = to_np(out)
    if layout == "bnhd":
        got = np.transpose(got, (0, 2, 1, 3))
    assert_close(got, ref, dtype, f"random order {dtype} {layout}")


@pytest.mark.parametrize("seed", range(10))
def test_random_tiles(seed):
    """Seeded random cases: a random permutation of n tokens, a tile dividing
    n (up to 768 tokens: several query units per tile past 256), any slide,
    a random memory row set or none, with or without a bias, both layouts,
    head dim 64/128, bf16 and fp32."""
    rng = np.random.default_rng(7000 + seed)
    tile = int(rng.integers(8, 769))
    ntiles = int(rng.integers(1, 7))
    n = tile * ntiles
    slide = int(rng.integers(-2 * n, 2 * n + 1))
    G = int(rng.integers(1, min(300, n) + 1)) if rng.random() < 0.7 else 0
    bias = float(rng.normal()) if G and rng.random() < 0.5 else 0.0
    D = int(rng.choice([64, 128]))
    dtype = "bf16" if rng.random() < 0.75 else "f32"
    layout = "bhnd" if rng.random() < 0.5 else "bnhd"
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    order = rng.permutation(n)
    idx = rng.choice(n, G, replace=False) if G else None
    log(f"random tiles seed={seed} n={n} tile={tile} slide={slide} G={G} bias={bias:.3f} "
        f"D={D} {dtype} {layout} B={B} H={H}")
    q, k, v = random_qkv((B, H, n, D), dtype, seed=8000 + seed)
    km = vm = None
    if G:
        km, vm = k[:, :, idx], v[:, :, idx]
    ref = O.curve_attention(q, k, v, order, tile, slide, km, vm, mem_logit_bias=bias)
    conv = (lambda x: x) if layout == "bhnd" else bhnd_to_bnhd
    qg, kg, vg = (to_gpu(conv(x), dtype) for x in (q, k, v))
    mem = S.gather_kv(kg, vg, _order(idx), layout=layout) if G else None
    out = S.curve_attn(qg, kg, vg, _order(order), tile, slide, mem=mem, mem_bias=bias,
                       layout=layout)
    torch.cuda.synchronize()
    got = to_np(out)
    if layout == "bnhd":
        got = np.transpose(got, (0, 2, 1, 3))
    assert_close(got, ref, dtype, f"random tiles {seed}")


@pytest.mark.parametrize("with_mem", [False, True])
def test_raster_order_is_row_window_attention(with_mem):
    # the same kernels through both address maps: results agree bit for bit
    n, tile, slide, B, H, D = 4096, 256, 77, 1, 3, 128
    log(f"raster order vs window_attn mem={with_mem}")
    q, k, v = random_qkv((B, H, n, D), "bf16", seed=11)
    qg, kg, vg = (to_gpu(x, "bf16") for x in (q, k, v))
    mem = S.pool_kv(kg, vg, (1, n), (1, 64)) if with_mem else None
    a = S.curve_attn(qg, kg, vg, _order(np.arange(n)), tile, slide, mem=mem)
    b = S.window_attn(qg, kg, vg, (1, n), (1, tile), (0, slide), mem=mem)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
def test_gather_kv(dtype, layout):
    B, H, n, D = 2, 3, 500, 128
    log(f"gather {dtype} {layout}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    shape = (B, H, n, D) if layout == "bhnd" else (B, n, H, D)
    k = torch.randn(shape, device="cuda", dtype=torch.float32).to(tdt)
    v = torch.randn(shape, device="cuda", dtype=torch.float32).to(tdt)
    idx = np.array([0, 499, 3, 3, 250, -7, 600], dtype=np.int32)   # duplicates, clamping
    ko, vo = S.gather_kv(k, v, _order(idx), layout=layout)
    torch.cuda.synchronize()
    sel = torch.from_numpy(np.clip(idx, 0, n - 1).astype(np.int64)).cuda()
    kb = k if layout == "bhnd" else k.transpose(1, 2)
    vb = v if layout == "bhnd" else v.transpose(1, 2)
    assert torch.equal(ko, kb.index_select(2, sel))
    assert torch.equal(vo, vb.index_select(2, sel))


@pytest.mark.parametrize("slide", [0, 128])
def test_hilbert_flux_shape(slide):
    # 128 x 128 tokens, 24 heads, tile 256 with an 8 x 8 central region: the
    # launch the benchmark times, with the library's own curve order and
    # region on the GPU (the oracle's only as the reference).  The output
    # starts NaN-filled; every element of every head must be written, and
    # three whole heads match the oracle.
    side, tile, B, H, D = 128, 256, 1, 24, 128
    n = side * side
    log(f"hilbert 128x128 slide {slide}")
    g = torch.Generator(device="cuda")
    g.manual_seed(21 + slide)
    qg, kg, vg = (torch.randn((B, H, n, D), generator=g, device="cuda").to(torch.bfloat16)
                  for _ in range(3))
    mem = S.gather_kv(kg, vg, _order(S.center_region_tokens((side, side), (8, 8))))
    out = torch.full_like(qg, float("nan"))
    S.curve_attn(qg, kg, vg, _order(S.hilbert_order(side)), tile, slide, mem=mem, out=out)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(out).any()), "unwritten output elements"
    reg = O.center_region((side, side), (8, 8))
    order = O.hilbert_order(side)
    for h in (0, 11, 23):
        q, k, v = (to_np(x[0:1, h:h + 1]) for x in (qg, kg, vg))
        ref = O.curve_attention(q, k, v, order, tile, slide, k[:, :, reg], v[:, :, reg])
        assert_close(to_np(out[0:1, h:h + 1]), ref, "bf16", f"flux hilbert head {h}")
