"""One step (pool of K/V, then window attention over the window and memory
keys) captured in a HIP graph per shift phase, replayed several times with
eager work and synchronisations between the replays: every replay equals the
eager step bit for bit (the kernels are deterministic), and the eager step
matches the oracle on sampled windows.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import assert_close, log, sample_windows, to_gpu, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_window_attention_amd")


def test_graph_replays_equal_eager_step():
    wl = W.FLUX1024
    log(f"graph step {wl.name}")
    q, k, v = W.make_qkv(wl)
    qg, kg, vg = (to_gpu(x, "bf16") for x in (q, k, v))
    B, H, n, D = qg.shape
    mem = tuple(torch.empty((B, H, wl.mem_tokens, D), dtype=torch.bfloat16, device=qg.device)
                for _ in range(2))
    out = torch.empty_like(qg)

    def step(phase, dst):
        shift = S.shift_for_block(phase, wl.schedule, wl.window)
        m = S.pool_kv(kg, vg, wl.grid, wl.pool, out=mem)
        S.window_attn(qg, kg, vg, wl.grid, wl.window, shift, mem=m, out=dst)

    phases = range(4)
    for ph in phases:  # eager warm-up: one-time launch set-up stays out of the graphs
        step(ph, out)
    torch.cuda.synchronize()
    graphs = []
    for ph in phases:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(ph, out)
        graphs.append(g)
    torch.cuda.synchronize()

    ref = torch.empty_like(qg)
    noise = torch.randn(1 << 20, device=qg.device)
    for rep in range(3):
        for ph in phases:
            out.zero_()
            torch.cuda.synchronize()
            graphs[ph].replay()
            noise.mul_(0.5).add_(1.0)  # unrelated eager work between replays
            torch.cuda.synchronize()
            step(ph, ref)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"replay {rep} of phase {ph} differs from eager"

    # the eager step of the last phase against the oracle (head 0, sampled windows)
    shift = S.shift_for_block(phases[-1], wl.schedule, wl.window)
    km = O.pool_mean(k[0:1, 0:1], wl.grid, wl.pool)[0, 0]
    vm = O.pool_mean(v[0:1, 0:1], wl.grid, wl.pool)[0, 0]
    nW = n // int(np.prod(wl.window))
    idx, exp = O.window_attention_head(q[0, 0], k[0, 0], v[0, 0], wl.grid, wl.window, shift,
                                       km, vm, windows=sample_windows(nW))
    got = to_np(ref[0, 0][torch.from_numpy(idx.reshape(-1)).to(ref.device)])
    assert_close(got.reshape(exp.shape), exp, "bf16", f"graph step {wl.name} shift {shift}")
