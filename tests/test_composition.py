"""The composition baseline that bench.py times against the fused kernel:
materialised roll + window partition, each window's keys concatenated with
the pooled memory, the library's unmodified dense kernel over the window
batches, then unpartition + unroll (BASA forum summary, "Overview" and "The
BASA Method": the method runs on existing dense attention backends)."""
import numpy as np
import pytest

import oracle as O
import workloads as W

torch = pytest.importorskip("torch")
bench = pytest.importorskip("bench")


@pytest.mark.parametrize("grid,window,shift", [
    ((8, 12), (4, 6), (1, 5)),
    ((8, 12), (4, 6), (-3, 13)),
    ((4, 6, 10), (2, 3, 5), (1, 2, 3)),
    ((16, 16), (16, 16), (0, 0)),
])
def test_window_permutation_matches_oracle_index(grid, window, shift):
    perm, inv = bench.window_permutation(grid, window, shift, "cpu")
    ref = O.window_token_index(grid, window, shift).reshape(-1)
    assert np.array_equal(perm.numpy(), ref)
    n = int(np.prod(grid))
    assert np.array_equal(perm[inv].numpy(), np.arange(n))


@pytest.mark.parametrize("grid,window,shift", [((8, 12), (4, 6), (1, 5)),
                                               ((4, 6, 10), (2, 3, 5), (3, -2, 7))])
def test_composition_index_matches_oracle_index(grid, window, shift):
    # row (b, j, h, r) of the window-batched tensor is token index[j, r] of
    # head (b, h); the inverse map puts every row back at its raster place
    B, H = 2, 3
    n = int(np.prod(grid))
    m = int(np.prod(window))
    fwd, inv = bench.composition_index(B, H, grid, window, shift, "cpu")
    index = O.window_token_index(grid, window, shift)
    nW = index.shape[0]
    f = fwd.numpy().reshape(B, nW, H, m)
    for b in range(B):
        for h in range(H):
            assert np.array_equal(f[b, :, h, :], (b * H + h) * n + index)
    assert np.array_equal(fwd[inv].numpy(), np.arange(B * H * n))


CASES = [
    # grid, window, pool, shift, heads
    ((32, 48), (16, 16), (8, 8), (8, 5), 6),
    ((6, 10, 26), (3, 5, 13), (3, 5, 2), (1, 3, 7), 4),
    ((16, 48), (16, 16), None, (8, 3), 3),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(len(CASES)))
def test_composition_matches_oracle(case):
    S = pytest.importorskip("sparse_window_attention_amd")
    from gpu_util import assert_close, log, random_qkv, to_gpu, to_np
    grid, window, pool, shift, H = CASES[case]
    n = int(np.prod(grid))
    log(f"composition vs oracle grid={grid} window={window} pool={pool}")
    q, k, v = random_qkv((2, H, n, 128), "bf16", seed=41 + case)
    qg, kg, vg = (to_gpu(x, "bf16") for x in (q, k, v))
    mem = S.pool_kv(kg, vg, grid, pool) if pool else None
    comp = bench.compose_attention(S, qg, kg, vg, mem, grid, window, shift)
    torch.cuda.synchronize()
    km = vm = None
    if pool:
        km, vm = O.pool_mean(k, grid, pool), O.pool_mean(v, grid, pool)
    ref = O.window_attention(q, k, v, grid, window, shift, km, vm)
    assert_close(to_np(comp), ref, "bf16", f"composition case {case}")


@pytest.mark.gpu
def test_composition_flux2048_matches_oracle():
    # the shape and memory the benchmark times the composition on: three
    # seeded heads checked whole at one phase of the schedule
    S = pytest.importorskip("sparse_window_attention_amd")
    from gpu_util import assert_close, log, make_full_inputs, to_np
    wl = W.FLUX2048_W16
    heads = [0, 11, 23]
    shift = S.shift_for_block(3, wl.schedule, wl.window)
    log(f"composition {wl.name} shift {shift}")
    (qg, kg, vg), exact = make_full_inputs(wl, heads)
    mem = S.pool_kv(kg, vg, wl.grid, wl.pool)
    comp = bench.compose_attention(S, qg, kg, vg, mem, wl.grid, wl.window, shift)
    torch.cuda.synchronize()
    for h in heads:
        q, k, v = (x[None, None] for x in exact[h])
        ref = O.window_attention(q, k, v, wl.grid, wl.window, shift,
                                 O.pool_mean(k, wl.grid, wl.pool), O.pool_mean(v, wl.grid, wl.pool))
        assert_close(to_np(comp[0, h]), ref[0, 0], "bf16", f"composition {wl.name} head {h}")
