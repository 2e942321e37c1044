"""Helpers for the GPU parity tests (HIP path through the C ABI vs the oracle)."""
import math
import sys

import numpy as np

import oracle as O
import workloads as W

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-5


def log(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def torch_dev():
    import torch
    return torch.device("cuda:0")


def to_gpu(x, dtype):
    """numpy float32 values (exact in dtype) -> GPU tensor of dtype."""
    import torch
    t = torch.from_numpy(np.array(x, dtype=np.float32, order="C"))   # a writable copy
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(torch_dev())


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    log(f"{what}: max abs {mx:.3e} mean abs {mean:.3e}")
    if dtype == "bf16":
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (what, mx, mean)
    else:
        assert mx <= F32_MAX_ABS, (what, mx, mean)
    return mx, mean


def random_qkv(shape, dtype, seed, values="iid"):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(3):
        x = rng.standard_normal(shape, dtype=np.float32)
        out.append(W.round_bf16(x) if dtype == "bf16" else x)
    return out


def bhnd_to_bnhd(x):
    return np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)))


def make_full_inputs(wl, exact_heads, variant=0):
    """GPU Q, K, V for all heads of ``wl``; ``exact_heads`` hold the seeded
    workload values (returned as numpy), the rest are filled on the GPU with
    other random values of the same distribution (heads are independent)."""
    import torch
    B, H, n, D = wl.batch, wl.heads, wl.n_tokens, wl.head_dim
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    g = torch.Generator(device=torch_dev())
    g.manual_seed(1234 + wl.seed)
    gpu = [torch.randn((B, H, n, D), generator=g, device=torch_dev(), dtype=torch.float32).to(tdt)
           for _ in range(3)]
    exact = {}
    for h in exact_heads:
        vals = [W.head_values(wl, t, h, variant) for t in range(3)]
        exact[h] = vals
        for t in range(3):
            x = torch.from_numpy(vals[t]).to(tdt).to(torch_dev())
            gpu[t][:, h] = x[None]
    return gpu, exact


def sample_windows(nW, k=4):
    picks = sorted({0, nW - 1, nW // 2, (nW * 3) // 7})
    return picks[:k] if len(picks) > k else picks


def random_geometry(seed, f32=True):
    """A seeded geometry within the API's contract: the window and the pool
    divide the grid on every axis, shifts anywhere (negative, past the
    window, past the grid), windows of up to 768 tokens (several query
    units per window past 256); bf16 only when ``f32`` is false."""
    rng = np.random.default_rng(seed)
    nd = int(rng.integers(2, 4))
    if nd == 2:
        window = (1024, 1)
        while window[0] * window[1] > 768:
            window = (int(rng.integers(2, 29)), int(rng.integers(2, 29)))
    else:
        window = (int(rng.integers(1, 5)), int(rng.integers(2, 9)), int(rng.integers(2, 13)))
    counts = tuple(int(rng.integers(1, 4)) for _ in window)
    grid = tuple(w * c for w, c in zip(window, counts))
    shift = tuple(int(rng.integers(-2 * w, 2 * w + 1)) for w in window)
    pool = None
    if rng.random() < 0.75:
        divs = [[d for d in range(1, g + 1) if g % d == 0] for g in grid]
        pool = tuple(int(rng.choice(d)) for d in divs)
    D = int(rng.choice([64, 128]))
    dtype = "bf16" if rng.random() < 0.75 or not f32 else "f32"
    layout = "bhnd" if rng.random() < 0.5 else "bnhd"
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    bias = float(np.log(np.prod(pool))) if pool is not None and rng.random() < 0.5 else 0.0
    return grid, window, shift, pool, D, dtype, layout, B, H, bias
