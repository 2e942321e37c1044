"""CPU oracle for the backward pass of shifted window attention with pooled
K/V memory.

TEST INFRASTRUCTURE ONLY (the same rule as basa_oracle: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it).  Plain numpy in float64; nothing is rounded.

What is differentiated is the forward of basa_oracle: for one (batch, head),
K_mem / V_mem are the means of K / V over the pool cells of the unshifted
grid; the grid is rolled by -shift and cut into windows; each window's
queries attend, under one softmax with scale alpha, to [window keys; memory
keys] (memory logits shifted by a constant bias); the outputs are rolled
back.  Sources: BASA forum summary, "The BASA Method" (shifted windows);
BASA discussion reply, the four parts of the method (pooled K/V memory);
Scale-Free Attention abstract (mean pooling under a shared softmax).  The
pages carry no backward pass; the training side of the method (the
dense-teacher adaptation on the BASA pages) needs one, and this is the
exact gradient of the forward above.

Per window, with S = alpha Q Kc^T + bias, P = softmax_row(S), O = P Vc:
    D_i   = sum_d dO_id O_id
    dP    = dO Vc^T
    dS    = P * (dP - D)          (row i of dP shifted by D_i)
    dQ    = alpha dS Kc
    dKc   = alpha dS^T Q
    dVc   = P^T dO
Each window key belongs to exactly one window, so its gradient is the
window's.  A memory key is seen by every window: its gradient is the sum
over windows.  Mean pooling passes dK_mem[g] / |cell g| to every token of
cell g, which adds to that token's own window gradient.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .basa_oracle import _as3, _f64, pool_mean, window_token_index


def attention_backward_rows(q, kc, vc, dout, scale: float, bias=None):
    """Gradients of O = softmax(scale q kc^T + bias) vc for one set of rows.

    Returns (dq, dkc, dvc, lse) where lse is the natural-log logsumexp of the
    scaled, biased logits of every row.
    """
    q, kc, vc, dout = _f64(q), _f64(kc), _f64(vc), _f64(dout)
    s = scale * (q @ kc.T)
    if bias is not None:
        s = s + bias[None, :]
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    den = e.sum(axis=1, keepdims=True)
    p = e / den
    lse = (mx + np.log(den))[:, 0]
    o = p @ vc
    d = np.sum(dout * o, axis=1, keepdims=True)
    dp = dout @ vc.T
    ds = p * (dp - d)
    dq = scale * (ds @ kc)
    dkc = scale * (ds.T @ q)
    dvc = p.T @ dout
    return dq, dkc, dvc, lse


def pool_backward(dmem, grid: Sequence[int], pool: Sequence[int]) -> np.ndarray:
    """Gradient of mean pooling: [G, D] cell gradients -> [n, D] token gradients
    (each token of cell g receives dmem[g] / |cell|), raster order."""
    dmem = _f64(dmem)
    T, Hg, Wg = _as3(grid, 1)
    pt, py, px = _as3(pool, 1)
    D = dmem.shape[-1]
    cells = dmem.reshape(T // pt, Hg // py, Wg // px, D) / float(pt * py * px)
    full = np.broadcast_to(cells[:, None, :, None, :, None, :],
                           (T // pt, pt, Hg // py, py, Wg // px, px, D))
    return np.ascontiguousarray(full).reshape(T * Hg * Wg, D)


def window_attention_backward_head(q, k, v, dout, grid, window, shift,
                                   pool: Optional[Sequence[int]] = None,
                                   scale: Optional[float] = None,
                                   mem_logit_bias: float = 0.0):
    """Backward of window_attention_head for one (batch, head).

    q, k, v, dout are [n, D].  With ``pool`` the memory is pooled from k, v
    (its gradient flows back into dk, dv).  Returns a dict with dq, dk, dv
    ([n, D], raster order), lse ([n], natural log, raster order) and, with a
    pool, dk_mem and dv_mem ([G, D], before the pooling backward).
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    n, D = q.shape
    alpha = 1.0 / math.sqrt(D) if scale is None else float(scale)
    index = window_token_index(grid, window, shift)          # [nW, m]
    nW, m = index.shape
    km = vm = None
    bias = None
    if pool is not None:
        km = pool_mean(k[None, None], grid, pool)[0, 0]
        vm = pool_mean(v[None, None], grid, pool)[0, 0]
        if mem_logit_bias:
            bias = np.concatenate([np.zeros(m), np.full(km.shape[0], mem_logit_bias)])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    lse = np.zeros(n)
    dkm = None if km is None else np.zeros_like(km)
    dvm = None if vm is None else np.zeros_like(vm)
    for j in range(nW):
        rows = index[j]
        kc, vc = k[rows], v[rows]
        if km is not None:
            kc = np.concatenate([kc, km], axis=0)
            vc = np.concatenate([vc, vm], axis=0)
        gq, gk, gv, l = attention_backward_rows(q[rows], kc, vc, dout[rows], alpha, bias)
        dq[rows] = gq
        dk[rows] += gk[:m]
        dv[rows] += gv[:m]
        lse[rows] = l
        if km is not None:
            dkm += gk[m:]
            dvm += gv[m:]
    res = {"dq": dq, "dk": dk, "dv": dv, "lse": lse}
    if km is not None:
        dk += pool_backward(dkm, grid, pool)
        dv += pool_backward(dvm, grid, pool)
        res["dk_mem"], res["dv_mem"] = dkm, dvm
    return res


def window_attention_backward(q, k, v, dout, grid, window, shift,
                              pool: Optional[Sequence[int]] = None,
                              scale: Optional[float] = None,
                              mem_logit_bias: float = 0.0):
    """window_attention_backward_head over [B, H, n, D]; returns a dict of
    stacked arrays (dq, dk, dv [B, H, n, D]; lse [B, H, n]; dk_mem, dv_mem
    [B, H, G, D] with a pool)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H = q.shape[:2]
    out = {}
    for b in range(B):
        for h in range(H):
            r = window_attention_backward_head(q[b, h], k[b, h], v[b, h], dout[b, h], grid,
                                               window, shift, pool, scale, mem_logit_bias)
            for key, val in r.items():
                if key not in out:
                    out[key] = np.zeros((B, H) + val.shape)
                out[key][b, h] = val
    return out
