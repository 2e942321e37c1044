"""Seeded synthetic workloads shared by the CPU oracle, the tests and the bench.

This module holds shapes and random-number recipes only: no step of the
attention method is computed here (no shift, window, pooling or softmax).
Both the oracle and the GPU path receive the arrays made here.

Workload shapes follow the DiT settings the BASA pages describe (FLUX image
and Wan video models, BASA forum summary, "Results"): token grids of 2D
images and 3D videos with multi-head attention of head dim 128. The pages
give no tensor values, so values are synthetic:

* ``iid``   -- N(0, 1) per element (float32 draw).
* ``field`` -- N(0, 1) plus a smooth spatial field, the sum of 8 random
  sinusoids over the grid with integer frequencies in [-3, 3] per axis (so
  the field is periodic on the torus and cyclic shifts keep it smooth),
  random phase, and per-channel weights drawn N(0, 1/8) and scaled by 0.5,
  giving each channel the RMS (0.354) of a sinusoid of amplitude 0.5.

bf16 workloads are rounded from the float32 draw with round-to-nearest-even
(torch CPU ``.to(torch.bfloat16)``).

Every (workload seed k, tensor t in {Q=0, K=1, V=2}, head h) pair has its own
numpy stream ``default_rng([k, t, h])`` (plus an optional ``variant`` for
rotated input sets), so a single head can be regenerated on its own.
"""
from __future__ import annotations

from dataclasses import dataclass, field as dc_field
from typing import Optional, Sequence, Tuple

import numpy as np

SCHED_NONE = 0
SCHED_ALTERNATE = 1
SCHED_FOUR_PHASE = 2

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    """One attention workload: shapes, schedule and value recipe."""

    name: str
    seed: int                      # workload seed index k
    batch: int
    heads: int
    head_dim: int
    grid: Tuple[int, ...]          # (Hg, Wg) or (T, Hg, Wg)
    window: Tuple[int, ...]
    pool: Optional[Tuple[int, ...]]  # None: no pooled memory
    schedule: int                  # SCHED_* used across blocks
    dtype: str                     # "bf16" | "f32"
    values: str                    # "iid" | "field"
    fixed_shift: Optional[Tuple[int, ...]] = None  # overrides the schedule
    blocks: int = 2                # blocks the schedule is exercised over
    note: str = ""

    @property
    def ndim(self) -> int:
        return len(self.grid)

    @property
    def n_tokens(self) -> int:
        return int(np.prod(self.grid))

    @property
    def window_tokens(self) -> int:
        return int(np.prod(self.window))

    @property
    def n_windows(self) -> int:
        return self.n_tokens // self.window_tokens

    @property
    def mem_tokens(self) -> int:
        if self.pool is None:
            return 0
        return int(np.prod([g // p for g, p in zip(self.grid, self.pool)]))

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The workloads.  Names say what they are; sizes are stated in full.
TINY = Workload(
    name="tiny_16x16_w8_f32", seed=0, batch=1, heads=1, head_dim=64,
    grid=(16, 16), window=(8, 8), pool=None, schedule=SCHED_NONE,
    dtype="f32", values="iid", fixed_shift=(4, 4), blocks=1,
    note="2D, 256 tokens, fixed cyclic shift (4,4), no memory, fp32")

FLUX1024 = Workload(
    name="flux1024_64x64_w16_pool4", seed=1, batch=1, heads=24, head_dim=128,
    grid=(64, 64), window=(16, 16), pool=(4, 4), schedule=SCHED_ALTERNATE,
    dtype="bf16", values="field", blocks=2,
    note="FLUX-like 1024px image: 4096 tokens, 256 pooled memory tokens")

FLUX2048_W16 = Workload(
    name="flux2048_128x128_w16_pool8", seed=2, batch=1, heads=24, head_dim=128,
    grid=(128, 128), window=(16, 16), pool=(8, 8), schedule=SCHED_FOUR_PHASE,
    dtype="bf16", values="field", blocks=4,
    note="FLUX-like 2048px image: 16384 tokens, window 16x16, 256 memory tokens")

FLUX2048_W32 = FLUX2048_W16.with_(
    name="flux2048_128x128_w32_pool8", window=(32, 32),
    note="FLUX-like 2048px image: 16384 tokens, window 32x32, 256 memory tokens")

WAN = Workload(
    name="wan_21x30x52_w7x10x13_pool3x5x4", seed=3, batch=1, heads=40,
    head_dim=128, grid=(21, 30, 52), window=(7, 10, 13), pool=(3, 5, 4),
    schedule=SCHED_ALTERNATE, dtype="bf16", values="field", blocks=2,
    note="Wan-like video: 32760 tokens, 910-token windows, 546 memory tokens")

WAN_G1638 = WAN.with_(
    name="wan_21x30x52_w7x10x13_pool1x5x4", pool=(1, 5, 4),
    note="Wan-like video with a (1,5,4) pool: 1638 memory tokens")

ULTRA = Workload(
    name="ultra_512x512_w32_pool8", seed=4, batch=1, heads=24, head_dim=128,
    grid=(512, 512), window=(32, 32), pool=(8, 8), schedule=SCHED_FOUR_PHASE,
    dtype="bf16", values="field", blocks=4,
    note="512x512 grid: 262144 tokens, 4096 memory tokens")

ALL = (TINY, FLUX1024, FLUX2048_W16, FLUX2048_W32, WAN, WAN_G1638, ULTRA)
BY_NAME = {w.name: w for w in ALL}


def _grid3(grid: Sequence[int]) -> Tuple[int, int, int]:
    return (1,) + tuple(grid) if len(grid) == 2 else tuple(grid)


def head_values_f32(wl: Workload, tensor: int, head: int, variant: int = 0,
                    values: Optional[str] = None) -> np.ndarray:
    """float32 [n, D] draw for one (tensor, head) of ``wl`` (batch shares it).

    ``variant`` > 0 selects an independent input set of the same recipe
    (used to rotate input sets through the caches when timing).
    """
    values = values or wl.values
    key = [wl.seed, tensor, head] + ([variant] if variant else [])
    rng = np.random.default_rng(key)
    n, d = wl.n_tokens, wl.head_dim
    x = rng.standard_normal((n, d), dtype=np.float32)
    if values == "iid":
        return x
    assert values == "field", values
    T, Hg, Wg = _grid3(wl.grid)
    nterm = 8
    while True:
        fr = rng.integers(-3, 4, size=(nterm, 3))
        if wl.ndim == 2:
            fr[:, 0] = 0
        if np.all(np.any(fr != 0, axis=1)):
            break
    phase = rng.uniform(0.0, 2.0 * np.pi, size=nterm)
    w = rng.standard_normal((nterm, d)) * np.sqrt(1.0 / nterm)
    t = np.arange(T, dtype=np.float64)[:, None, None] / T
    y = np.arange(Hg, dtype=np.float64)[None, :, None] / Hg
    xx = np.arange(Wg, dtype=np.float64)[None, None, :] / Wg
    waves = np.empty((n, nterm), dtype=np.float64)
    for k in range(nterm):
        arg = 2.0 * np.pi * (fr[k, 0] * t + fr[k, 1] * y + fr[k, 2] * xx) + phase[k]
        waves[:, k] = np.sin(arg).reshape(-1)
    fieldv = 0.5 * (waves @ w)
    return (x.astype(np.float64) + fieldv).astype(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (RNE) and return the bf16 values as float32."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).float().numpy()


def head_values(wl: Workload, tensor: int, head: int, variant: int = 0,
                values: Optional[str] = None) -> np.ndarray:
    """[n, D] float32 holding exactly the values the GPU receives."""
    x = head_values_f32(wl, tensor, head, variant, values)
    return round_bf16(x) if wl.dtype == "bf16" else x


def make_qkv(wl: Workload, heads: Optional[Sequence[int]] = None,
             variant: int = 0, values: Optional[str] = None):
    """Q, K, V as float32 arrays [B, len(heads), n, D] (BHND layout).

    Values are exactly representable in the workload dtype.  All batch
    entries share the same draw.
    """
    heads = list(range(wl.heads)) if heads is None else list(heads)
    out = []
    for t in (TENSOR_Q, TENSOR_K, TENSOR_V):
        per_head = np.stack([head_values(wl, t, h, variant, values) for h in heads])
        out.append(np.ascontiguousarray(
            np.broadcast_to(per_head[None], (wl.batch,) + per_head.shape)))
    return tuple(out)


def to_torch(x: np.ndarray, dtype: str):
    """numpy float32 -> torch CPU tensor of the workload dtype (exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t
