"""Pins of the backward oracle.

The oracle's gradients come from the textbook softmax-attention backward
written out (oracle/basa_backward.py).  They are checked here against
torch.autograd in float64 applied to an independent torch statement of the
forward (roll, partition, concatenated memory, softmax, unpartition; pooling
by reshape-mean), and against finite differences of the numpy forward oracle
on tiny cases.
"""
import math

import numpy as np
import pytest

import oracle as O

torch = pytest.importorskip("torch")


def torch_forward(q, k, v, grid, window, shift, pool, bias):
    """[n, D] tensors of one head -> output [n, D]; differentiable."""
    g = list(grid) if len(grid) == 3 else [1] + list(grid)
    w = list(window) if len(window) == 3 else [1] + list(window)
    s = list(shift) if len(shift) == 3 else [0] + list(shift)
    n, D = q.shape
    alpha = 1.0 / math.sqrt(D)

    def part(x):
        x = x.reshape(*g, D)
        x = torch.roll(x, shifts=[-t for t in s], dims=(0, 1, 2))
        x = x.reshape(g[0] // w[0], w[0], g[1] // w[1], w[1], g[2] // w[2], w[2], D)
        return x.permute(0, 2, 4, 1, 3, 5, 6).reshape(-1, w[0] * w[1] * w[2], D)

    qw, kw, vw = part(q), part(k), part(v)
    nW, m = qw.shape[:2]
    if pool is not None:
        p = list(pool) if len(pool) == 3 else [1] + list(pool)
        def pooled(x):
            x = x.reshape(g[0] // p[0], p[0], g[1] // p[1], p[1], g[2] // p[2], p[2], D)
            return x.mean(dim=(1, 3, 5)).reshape(-1, D)
        km, vm = pooled(k), pooled(v)
        G = km.shape[0]
        kw = torch.cat([kw, km.unsqueeze(0).expand(nW, G, D)], dim=1)
        vw = torch.cat([vw, vm.unsqueeze(0).expand(nW, G, D)], dim=1)
    logits = alpha * qw @ kw.transpose(1, 2)
    if pool is not None and bias:
        logits = logits + torch.cat([torch.zeros(m, dtype=q.dtype),
                                     torch.full((G,), bias, dtype=q.dtype)])
    ow = torch.softmax(logits, dim=-1) @ vw
    ow = ow.reshape(g[0] // w[0], g[1] // w[1], g[2] // w[2], w[0], w[1], w[2], D)
    ow = ow.permute(0, 3, 1, 4, 2, 5, 6).reshape(*g, D)
    return torch.roll(ow, shifts=s, dims=(0, 1, 2)).reshape(n, D)


CASES = [
    # grid, window, shift, pool, bias
    ((4, 6), (2, 3), (1, 2), None, 0.0),
    ((4, 6), (2, 3), (1, 2), (2, 3), 0.0),
    ((6, 4), (3, 2), (-1, 5), (3, 2), math.log(6.0)),
    ((2, 4, 6), (1, 2, 3), (1, 1, 2), (2, 2, 3), 0.0),
    ((4, 4), (4, 4), (0, 0), (4, 4), 0.5),
    ((4, 6), (2, 3), (0, 0), (1, 1), 0.0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_matches_autograd(case):
    grid, window, shift, pool, bias = CASES[case]
    n, D = int(np.prod(grid)), 8
    rng = np.random.default_rng(case)
    q, k, v, do = (rng.standard_normal((n, D)) for _ in range(4))
    ref = O.window_attention_backward_head(q, k, v, do, grid, window, shift, pool,
                                           mem_logit_bias=bias)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch_forward(tq, tk, tv, grid, window, shift, pool, bias)
    out.backward(torch.tensor(do))
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(ref[name], t.grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=name)
    # the forward the backward differentiates is the forward oracle
    km = vm = None
    if pool is not None:
        km = O.pool_mean(k[None, None], grid, pool)[0, 0]
        vm = O.pool_mean(v[None, None], grid, pool)[0, 0]
    fwd = O.window_attention(q[None, None], k[None, None], v[None, None], grid, window, shift,
                             None if km is None else km[None, None],
                             None if vm is None else vm[None, None], mem_logit_bias=bias)
    np.testing.assert_allclose(fwd[0, 0], out.detach().numpy(), rtol=1e-12, atol=1e-12)


def test_backward_finite_differences():
    grid, window, shift, pool = (4, 4), (2, 2), (1, 1), (2, 2)
    n, D = 16, 4
    rng = np.random.default_rng(7)
    q, k, v, do = (rng.standard_normal((n, D)) for _ in range(4))

    def loss(qq, kk, vv):
        km = O.pool_mean(kk[None, None], grid, pool)
        vm = O.pool_mean(vv[None, None], grid, pool)
        o = O.window_attention(qq[None, None], kk[None, None], vv[None, None], grid, window,
                               shift, km, vm)[0, 0]
        return float(np.sum(o * do))

    ref = O.window_attention_backward_head(q, k, v, do, grid, window, shift, pool)
    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        for (i, d) in [(0, 0), (5, 3), (15, 1), (10, 2)]:
            xp, xm = x.copy(), x.copy()
            xp[i, d] += eps
            xm[i, d] -= eps
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - ref[name][i, d]) < 1e-7, (name, i, d, fd, ref[name][i, d])


def test_lse_and_memory_gradient_closed_forms():
    # one window covering the grid, pool = whole grid: G = 1, and the memory
    # key's gradient is the sum of the gradients its pooled value stands for
    grid, window, shift, pool = (2, 3), (2, 3), (0, 0), (2, 3)
    n, D = 6, 5
    rng = np.random.default_rng(3)
    q, k, v, do = (rng.standard_normal((n, D)) for _ in range(4))
    r = O.window_attention_backward_head(q, k, v, do, grid, window, shift, pool)
    alpha = 1 / math.sqrt(D)
    km = k.mean(axis=0, keepdims=True)
    logits = alpha * q @ np.concatenate([k, km]).T
    np.testing.assert_allclose(r["lse"], np.log(np.exp(logits).sum(axis=1)), rtol=1e-12)
    # pooled gradient spreads evenly: dk = dk_window + dk_mem / n
    rr = O.attention_backward_rows(q, np.concatenate([k, km]), np.concatenate([v, v.mean(0, keepdims=True)]), do, alpha)
    np.testing.assert_allclose(r["dk"], rr[1][:n] + rr[1][n:] / n, rtol=1e-12)
    np.testing.assert_allclose(r["dv"], rr[2][:n] + rr[2][n:] / n, rtol=1e-12)
