"""The seeded synthetic inputs: deterministic, drawn per (tensor, head) so a
single head can be regenerated alone, exactly representable in the workload
dtype (bf16 by round-to-nearest-even), and, for the "field" recipe, noise
plus a sum of sinusoids with integer frequencies on the grid (so the field
has zero mean over every channel and is periodic on the torus).  CPU only.
"""
import numpy as np
import pytest

import workloads as W

torch = pytest.importorskip("torch")


def test_deterministic():
    wl = W.FLUX1024
    a = W.head_values(wl, W.TENSOR_K, 3)
    b = W.head_values(wl, W.TENSOR_K, 3)
    assert a.dtype == np.float32 and a.shape == (wl.n_tokens, wl.head_dim)
    assert np.array_equal(a, b)


def test_one_head_regenerates_alone():
    wl = W.FLUX1024
    q, k, v = W.make_qkv(wl, heads=[0, 5, 23])
    for t, x in enumerate((q, k, v)):
        assert x.shape == (wl.batch, 3, wl.n_tokens, wl.head_dim)
        for j, h in enumerate((0, 5, 23)):
            assert np.array_equal(x[0, j], W.head_values(wl, t, h))


def test_draws_are_independent():
    wl = W.FLUX1024
    base = W.head_values_f32(wl, W.TENSOR_Q, 0, values="iid").ravel()
    others = [W.head_values_f32(wl, W.TENSOR_K, 0, values="iid"),
              W.head_values_f32(wl, W.TENSOR_Q, 1, values="iid"),
              W.head_values_f32(wl, W.TENSOR_Q, 0, variant=1, values="iid"),
              W.head_values_f32(W.FLUX2048_W16, W.TENSOR_Q, 0, values="iid")[:wl.n_tokens]]
    for o in others:
        r = np.corrcoef(base, o.ravel())[0, 1]
        assert abs(r) < 0.01, r


def test_values_exact_in_dtype():
    for wl in (W.FLUX1024, W.WAN):
        x = W.head_values(wl, W.TENSOR_V, 2)
        bits = x.view(np.uint32)
        assert np.all(bits & 0xFFFF == 0), "not a bf16 value"
    tiny = W.head_values(W.TINY, W.TENSOR_Q, 0)
    assert np.array_equal(tiny, W.head_values_f32(W.TINY, W.TENSOR_Q, 0))


def test_bf16_rounding_is_nearest_even():
    one = 1.0
    ulp = 2.0 ** -7                      # bf16 spacing in [1, 2)
    x = np.array([one + ulp / 2,         # tie -> even (1.0)
                  one + 3 * ulp / 2,     # tie -> even (1 + 2 ulp)
                  one + ulp / 2 + 2 ** -20,  # above the tie -> up
                  -(one + ulp / 2)], dtype=np.float32)
    got = W.round_bf16(x)
    assert got.tolist() == [1.0, one + 2 * ulp, one + ulp, -1.0]


@pytest.mark.parametrize("wl", [W.FLUX1024, W.WAN], ids=lambda w: w.name)
def test_field_is_a_zero_mean_torus_field(wl):
    # same generator key: the "field" draw is the "iid" draw plus the field
    noise = W.head_values_f32(wl, W.TENSOR_K, 1, values="iid").astype(np.float64)
    total = W.head_values_f32(wl, W.TENSOR_K, 1, values="field").astype(np.float64)
    field = total - noise
    # integer frequencies, not all zero: every channel sums to zero over the grid
    rms = np.sqrt(np.mean(field ** 2))
    assert np.max(np.abs(field.mean(axis=0))) < 1e-5 * max(rms, 1.0)
    # 0.5-amplitude sinusoids with unit total weight variance: RMS near 0.354
    assert 0.15 < rms < 0.6, rms
    # periodic on the torus: the field is a band-limited sum of sinusoids with
    # |frequency| <= 3 per axis, so its DFT along each axis has no energy
    # above the third harmonic (a non-periodic field would leak into them)
    grid = (1,) + tuple(wl.grid) if len(wl.grid) == 2 else tuple(wl.grid)
    f = field.reshape(grid + (wl.head_dim,))
    spec = np.abs(np.fft.fftn(f, axes=(0, 1, 2))) ** 2
    keep = np.zeros(grid, dtype=bool)
    idx = [np.r_[0:4, n - 3:n] if n > 7 else np.arange(n) for n in grid]
    keep[np.ix_(*idx)] = True
    outside = spec[~keep].sum()
    assert outside < 1e-12 * spec.sum(), outside / spec.sum()
