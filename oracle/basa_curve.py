"""CPU oracle for attention inside tiles of a token order -- Hilbert-curve
tiles (HilbertA catalogue record, abstract: tokens reordered along a Hilbert
curve, attention inside contiguous tiles of that order, a sliding schedule
across layers, a small central region shared by every tile).

TEST INFRASTRUCTURE ONLY (the rule of basa_oracle applies).  numpy, float64.

Readings taken (the page is an abstract; none of these is fixed by it):
* The curve is the standard Hilbert curve on a 2^k x 2^k grid, from (0, 0)
  to (side-1, 0), built here from its self-similarity.
* A tile is `tile` consecutive curve positions; sliding by s moves every
  tile s positions along the curve, cyclically.
* The shared central region is a block of tokens at the grid centre whose
  keys and values are appended to every tile's keys under one softmax (a
  region token inside a tile then appears twice among that tile's keys).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .basa_oracle import _f64, _softmax_attend


def hilbert_curve_xy(side: int):
    """Points (x, y) of the Hilbert curve over a side x side grid, in curve
    order.  The curve of side 2s runs through the four s x s quadrants in the
    order lower-left, upper-left, upper-right, lower-right; each quadrant is
    the side-s curve, transposed in the lower-left, translated in the upper
    two, reflected across the anti-diagonal in the lower-right, so that the
    pieces join end to start."""
    if side < 1 or side & (side - 1):
        raise ValueError("side must be a power of two")
    if side == 1:
        return [(0, 0)]
    s = side // 2
    sub = hilbert_curve_xy(s)
    pts = [(y, x) for (x, y) in sub]
    pts += [(x, y + s) for (x, y) in sub]
    pts += [(x + s, y + s) for (x, y) in sub]
    pts += [(2 * s - 1 - y, s - 1 - x) for (x, y) in sub]
    return pts


def hilbert_order(side: int) -> np.ndarray:
    """Raster index y*side + x of every curve position."""
    return np.array([y * side + x for (x, y) in hilbert_curve_xy(side)], dtype=np.int64)


def center_region(grid: Sequence[int], size: Sequence[int]) -> np.ndarray:
    """Raster indices of the size[0] x size[1] block at the centre of a 2-D grid
    (first row and column at (grid - size) // 2), raster order."""
    Hg, Wg = grid
    ch, cw = size
    y0, x0 = (Hg - ch) // 2, (Wg - cw) // 2
    return np.array([(y0 + i) * Wg + (x0 + j) for i in range(ch) for j in range(cw)],
                    dtype=np.int64)


def curve_attention(q, k, v, order, tile: int, slide: int, k_mem=None, v_mem=None,
                    scale: Optional[float] = None, mem_logit_bias: float = 0.0):
    """[B, H, n, D] -> [B, H, n, D]: tile j holds the tokens
    order[(j*tile + slide + r) mod n], r < tile; each query attends to its
    tile's keys followed by the memory keys (per (b, h)) under one softmax."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    order = np.asarray(order, dtype=np.int64)
    B, H, n, D = q.shape
    if n % tile:
        raise ValueError("tile must divide n")
    alpha = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            km = None if k_mem is None else _f64(k_mem)[b, h]
            vm = None if v_mem is None else _f64(v_mem)[b, h]
            bias = None
            if km is not None and mem_logit_bias:
                bias = np.concatenate([np.zeros(tile), np.full(km.shape[0], mem_logit_bias)])
            for j in range(n // tile):
                idx = order[(j * tile + slide + np.arange(tile)) % n]
                kc, vc = k[b, h][idx], v[b, h][idx]
                if km is not None:
                    kc = np.concatenate([kc, km])
                    vc = np.concatenate([vc, vm])
                out[b, h][idx] = _softmax_attend(q[b, h][idx], kc, vc, alpha, bias)
    return out


def curve_attention_bruteforce(q, k, v, order, tile: int, slide: int, k_mem=None, v_mem=None,
                               scale: Optional[float] = None):
    """The same result from its definition: full attention over [K; K_mem]
    with key j kept for query i when both lie in the same tile (tile of a
    token = ((curve position - slide) mod n) // tile) or j is a memory key."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    order = np.asarray(order, dtype=np.int64)
    B, H, n, D = q.shape
    alpha = 1.0 / math.sqrt(D) if scale is None else float(scale)
    pos = np.empty(n, dtype=np.int64)
    pos[order] = np.arange(n)
    tid = ((pos - slide) % n) // tile
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            kc, vc = k[b, h], v[b, h]
            G = 0
            if k_mem is not None:
                kc = np.concatenate([kc, _f64(k_mem)[b, h]])
                vc = np.concatenate([vc, _f64(v_mem)[b, h]])
                G = k_mem.shape[2]
            s = alpha * q[b, h] @ kc.T
            allowed = np.concatenate([tid[:, None] == tid[None, :], np.ones((n, G), bool)], axis=1)
            s = np.where(allowed, s, -np.inf)
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[b, h] = p @ vc
    return out
