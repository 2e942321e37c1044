"""The composition baseline (materialised roll + partition, attention over
window-contiguous tensors, unpartition + unroll) that bench.py times against
the fused kernel."""
import numpy as np
import pytest

import oracle as O

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


@pytest.mark.gpu
@pytest.mark.parametrize("grid,window,pool,shift", [
    ((32, 48), (16, 16), (8, 8), (8, 5)),
    ((6, 10, 26), (3, 5, 13), (3, 5, 2), (1, 3, 7)),
    ((128, 128), (16, 16), (8, 8), (8, 8)),     # the FLUX-2048 grid the benchmark times
])
def test_composition_equals_fused(grid, window, pool, shift):
    S = pytest.importorskip("sparse_window_attention_amd")
    from gpu_util import log, random_qkv, to_gpu
    n = int(np.prod(grid))
    log(f"composition vs fused grid={grid} window={window}")
    q, k, v = random_qkv((1, 6, n, 128), "bf16", seed=41)
    qg, kg, vg = (to_gpu(x, "bf16") for x in (q, k, v))
    mem = S.pool_kv(kg, vg, grid, pool)
    fused = S.window_attn(qg, kg, vg, grid, window, shift, mem=mem)
    comp = bench.compose_attention(S, qg, kg, vg, mem, grid, window, shift)
    torch.cuda.synchronize()
    assert torch.equal(fused, comp)
