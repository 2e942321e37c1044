"""CPU oracle for shifted local window attention with pooled K/V memory.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never does, and this
module imports nothing from it.

Everything is plain numpy in float64 on exact upcasts of the inputs; nothing
is rounded.  Sources (the web pages on BASA and related methods):

* BASA forum summary (zhichai.net English mirror of "BASA: Backend-Agnostic
  Sparse Attention for Fast High-Resolution Diffusion Transformers"),
  sections "Summary" and "The BASA Method": visual self-attention is replaced
  by attention inside local windows of the token grid, and the window
  partition is shifted from one DiT block to the next in a structured way so
  that tokens cut apart by a window boundary meet in a later block.
* BASA discussion reply (zhichai.net topic reply), paragraph listing the
  method's four parts: shifted-window sparse attention plus a global memory
  built by pooling K and V, because shifted windows alone stay local.
* Scale-Free Attention abstract (artificialintelbulletin.com): distant
  regions are summarised by mean pooling and attended under one shared
  softmax with the local tokens.
* BASA discussion reply, paragraph on the complexity: full attention costs
  O(n^2), window attention O(n*m), so the ideal speedup is n/m.

Readings taken where the pages are silent (each is a convention, so the
pages cannot pin it; the tests pin the code to the reading):

* Shift direction: the grid is rolled by -s before partitioning, so window j
  along an axis holds the tokens at positions j*w + s ... j*w + s + w - 1
  (mod the grid size).  Token p lies in window floor(((p - s) mod N) / w).
* Tokens wrapped around the grid edge by the roll are not masked: they
  attend to each other inside their window (a cyclic shift).
* The memory pools the unshifted grid, so it is independent of the shift
  and shared by every window.  Every window sees all memory tokens,
  including the summary of its own tokens.
* One softmax scale 1/sqrt(D) for window and memory logits alike; no
  token-count correction on memory logits unless ``mem_logit_bias`` is
  given (the Scale-Free Attention abstract names such a correction without
  defining it; the reading here adds ln(pool cell size) to memory logits).
* Shift schedules: ALTERNATE uses no shift on even blocks and floor(w/2) on
  odd ones; FOUR_PHASE counts in binary over the axes (bit i of the phase
  block mod 2^ndim shifts axis i by floor(w_i/2)).

Array conventions: Q, K, V are [B, H, n, D] with tokens in raster order of
the grid, idx = (t*Hg + y)*Wg + x; 2D grids are (Hg, Wg) and act as T = 1.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

SCHED_NONE = 0
SCHED_ALTERNATE = 1
SCHED_FOUR_PHASE = 2


def _as3(v: Sequence[int], fill: int) -> Tuple[int, int, int]:
    v = tuple(int(a) for a in v)
    if len(v) == 2:
        return (fill,) + v
    if len(v) == 3:
        return v
    raise ValueError("grid/window/shift/pool must have 2 or 3 entries")


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Shift schedule (BASA forum summary, "The BASA Method": a structured shift of
# the window partition that changes from block to block).
# ---------------------------------------------------------------------------
def shift_for_block(block: int, schedule: int, window: Sequence[int]) -> Tuple[int, ...]:
    """Shift of the window partition used by DiT block ``block``.

    NONE: always zero.  ALTERNATE: zero on even blocks, floor(w/2) per axis on
    odd blocks.  FOUR_PHASE: phase = block mod 2^ndim; axis i is shifted by
    floor(w_i/2) when bit i of the phase is set (2D: (0,0), (w/2,0), (0,w/2),
    (w/2,w/2)).
    """
    if block < 0:
        raise ValueError("block index must be >= 0")
    half = [w // 2 for w in window]
    if schedule == SCHED_NONE:
        return tuple(0 for _ in window)
    if schedule == SCHED_ALTERNATE:
        return tuple(half) if block % 2 == 1 else tuple(0 for _ in window)
    if schedule == SCHED_FOUR_PHASE:
        phase = block % (1 << len(window))
        return tuple(half[i] if (phase >> i) & 1 else 0 for i in range(len(window)))
    raise ValueError("unknown schedule")


# ---------------------------------------------------------------------------
# Pooled K/V memory (BASA discussion reply, four-parts paragraph: a global
# memory made by pooling K/V; Scale-Free Attention abstract: mean pooling).
# ---------------------------------------------------------------------------
def mem_tokens(grid: Sequence[int], pool: Sequence[int]) -> int:
    g3, p3 = _as3(grid, 1), _as3(pool, 1)
    for g, p in zip(g3, p3):
        if p <= 0 or g % p:
            raise ValueError("pool must divide the grid")
    return int(np.prod([g // p for g, p in zip(g3, p3)]))


def pool_mean(x, grid: Sequence[int], pool: Sequence[int]) -> np.ndarray:
    """Mean of ``x`` [B, H, n, D] over each pool cell of the unshifted grid.

    Returns [B, H, G, D], memory tokens in raster order of the pooled grid.
    """
    x = _f64(x)
    B, H, n, D = x.shape
    T, Hg, Wg = _as3(grid, 1)
    pt, py, px = _as3(pool, 1)
    if n != T * Hg * Wg:
        raise ValueError("token count does not match the grid")
    mem_tokens(grid, pool)
    cells = x.reshape(B, H, T // pt, pt, Hg // py, py, Wg // px, px, D)
    m = cells.mean(axis=(3, 5, 7))
    return m.reshape(B, H, -1, D)


# ---------------------------------------------------------------------------
# Shifted window attention, step by step as the BASA pages describe it:
# shift the grid, cut it into windows, attend inside each window (with the
# pooled memory appended to each window's keys under the same softmax), then
# put the tokens back and undo the shift.
# ---------------------------------------------------------------------------
def _roll_grid(x: np.ndarray, grid3, shift3, sign: int) -> np.ndarray:
    """x [..., n, D]: np.roll over the grid axes by sign*shift."""
    lead = x.shape[:-2]
    D = x.shape[-1]
    g = x.reshape(lead + tuple(grid3) + (D,))
    axes = tuple(range(len(lead), len(lead) + 3))
    g = np.roll(g, shift=tuple(sign * s for s in shift3), axis=axes)
    return g.reshape(lead + (-1, D))


def _partition(x: np.ndarray, grid3, win3) -> np.ndarray:
    """x [..., n, D] (raster) -> [..., nW, m, D], windows and tokens raster."""
    lead = x.shape[:-2]
    D = x.shape[-1]
    T, Hg, Wg = grid3
    wt, wy, wx = win3
    L = len(lead)
    g = x.reshape(lead + (T // wt, wt, Hg // wy, wy, Wg // wx, wx, D))
    perm = tuple(range(L)) + (L, L + 2, L + 4, L + 1, L + 3, L + 5, L + 6)
    g = g.transpose(perm)
    return g.reshape(lead + (-1, wt * wy * wx, D))


def _unpartition(x: np.ndarray, grid3, win3) -> np.ndarray:
    """Inverse of ``_partition``: [..., nW, m, D] -> [..., n, D]."""
    lead = x.shape[:-3]
    D = x.shape[-1]
    T, Hg, Wg = grid3
    wt, wy, wx = win3
    L = len(lead)
    g = x.reshape(lead + (T // wt, Hg // wy, Wg // wx, wt, wy, wx, D))
    perm = tuple(range(L)) + (L, L + 3, L + 1, L + 4, L + 2, L + 5, L + 6)
    g = g.transpose(perm)
    return g.reshape(lead + (-1, D))


def _softmax_attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                    bias: Optional[np.ndarray] = None) -> np.ndarray:
    """softmax(scale * q k^T + bias) v for one set of rows (fp64)."""
    s = scale * (q @ k.T)
    if bias is not None:
        s = s + bias[None, :]
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


def _check_geometry(grid3, win3):
    for g, w in zip(grid3, win3):
        if w <= 0 or g <= 0 or g % w:
            raise ValueError("window must divide the grid")


def window_token_index(grid: Sequence[int], window: Sequence[int],
                       shift: Sequence[int]) -> np.ndarray:
    """[nW, m] raster index of each (window, slot) after shift + partition.

    Obtained by pushing the token index itself through the same roll and
    partition steps the values go through.
    """
    grid3, win3 = _as3(grid, 1), _as3(window, 1)
    shift3 = _as3(shift, 0)
    _check_geometry(grid3, win3)
    idx = np.arange(int(np.prod(grid3)), dtype=np.int64).reshape(-1, 1)
    r = _roll_grid(idx, grid3, shift3, -1)
    return _partition(r, grid3, win3)[..., 0]


def window_attention_head(q, k, v, grid, window, shift, k_mem=None, v_mem=None,
                          scale: Optional[float] = None,
                          windows: Optional[Iterable[int]] = None,
                          mem_logit_bias: float = 0.0):
    """Shifted window attention for one (batch, head): q, k, v are [n, D].

    Returns (index [len(windows), m], out [len(windows), m, D]): the raster
    index of every query row computed and its output.  ``windows`` selects
    windows of the shifted partition (all by default), so large grids can be
    checked on a sample of windows.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, D = q.shape
    grid3, win3 = _as3(grid, 1), _as3(window, 1)
    shift3 = _as3(shift, 0)
    _check_geometry(grid3, win3)
    if n != int(np.prod(grid3)):
        raise ValueError("token count does not match the grid")
    if (k_mem is None) != (v_mem is None):
        raise ValueError("k_mem and v_mem go together")
    alpha = 1.0 / math.sqrt(D) if scale is None else float(scale)

    # step 1: cyclic shift of the grid (roll by -s)
    qr = _roll_grid(q, grid3, shift3, -1)
    kr = _roll_grid(k, grid3, shift3, -1)
    vr = _roll_grid(v, grid3, shift3, -1)
    # step 2: partition into non-overlapping windows
    qw = _partition(qr, grid3, win3)
    kw = _partition(kr, grid3, win3)
    vw = _partition(vr, grid3, win3)
    index = window_token_index(grid, window, shift)
    nW, m = index.shape
    sel = list(range(nW)) if windows is None else [int(j) for j in windows]

    bias = None
    if k_mem is not None:
        k_mem, v_mem = _f64(k_mem), _f64(v_mem)
        if mem_logit_bias:
            bias = np.concatenate([np.zeros(m), np.full(k_mem.shape[0], mem_logit_bias)])

    # step 3: dense softmax attention inside each window, memory keys
    # appended to the window's keys under the same softmax
    outs = np.empty((len(sel), m, D), dtype=np.float64)
    for i, j in enumerate(sel):
        kc, vc = kw[j], vw[j]
        if k_mem is not None:
            kc = np.concatenate([kc, k_mem], axis=0)
            vc = np.concatenate([vc, v_mem], axis=0)
        outs[i] = _softmax_attend(qw[j], kc, vc, alpha, bias)
    return index[sel], outs


def window_attention(q, k, v, grid, window, shift, k_mem=None, v_mem=None,
                     scale: Optional[float] = None, mem_logit_bias: float = 0.0):
    """Shifted window attention over [B, H, n, D]; output [B, H, n, D] fp64.

    Steps: roll by -shift, partition, per-window softmax attention over
    [window keys; memory keys], unpartition, roll by +shift.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n, D = q.shape
    grid3, win3 = _as3(grid, 1), _as3(window, 1)
    shift3 = _as3(shift, 0)
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            km = None if k_mem is None else k_mem[b][h]
            vm = None if v_mem is None else v_mem[b][h]
            _, ow = window_attention_head(q[b, h], k[b, h], v[b, h], grid, window,
                                          shift, km, vm, scale,
                                          mem_logit_bias=mem_logit_bias)
            # step 4: undo the partition, then undo the shift
            orr = _unpartition(ow, grid3, win3)
            out[b, h] = _roll_grid(orr, grid3, shift3, +1)
    return out


# ---------------------------------------------------------------------------
# The same result from its plain definition: full attention over the
# concatenated keys [K; K_mem] with a block mask that keeps a key only when
# it is a memory key or lies in the query's (shifted) window.
# ---------------------------------------------------------------------------
def window_id(grid: Sequence[int], window: Sequence[int], shift: Sequence[int]) -> np.ndarray:
    """[n] window id of every raster token under the shifted partition."""
    grid3, win3 = _as3(grid, 1), _as3(window, 1)
    shift3 = _as3(shift, 0)
    T, Hg, Wg = grid3
    ids = np.empty(T * Hg * Wg, dtype=np.int64)
    nwy, nwx = Hg // win3[1], Wg // win3[2]
    for t in range(T):
        ct = ((t - shift3[0]) % T) // win3[0]
        for y in range(Hg):
            cy = ((y - shift3[1]) % Hg) // win3[1]
            for x in range(Wg):
                cx = ((x - shift3[2]) % Wg) // win3[2]
                ids[(t * Hg + y) * Wg + x] = (ct * nwy + cy) * nwx + cx
    return ids


def masked_attention_bruteforce(q, k, v, grid, window, shift, k_mem=None,
                                v_mem=None, scale: Optional[float] = None,
                                mem_logit_bias: float = 0.0):
    """softmax(alpha [Q][K; K_mem]^T + M) [V; V_mem] with the block mask M.

    M[i, j] = 0 when j is a memory key or window(i) == window(j), else -inf.
    Written with no roll and no reshape; O(n^2) -- tiny grids only.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n, D = q.shape
    alpha = 1.0 / math.sqrt(D) if scale is None else float(scale)
    wid = window_id(grid, window, shift)
    same = wid[:, None] == wid[None, :]
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            kc, vc = k[b, h], v[b, h]
            keep = same
            bias = np.zeros((n, n))
            if k_mem is not None:
                G = np.shape(k_mem)[2]
                kc = np.concatenate([kc, _f64(k_mem[b][h])], axis=0)
                vc = np.concatenate([vc, _f64(v_mem[b][h])], axis=0)
                keep = np.concatenate([same, np.ones((n, G), dtype=bool)], axis=1)
                bias = np.concatenate([bias, np.full((n, G), mem_logit_bias)], axis=1)
            s = alpha * (q[b, h] @ kc.T) + bias
            s = np.where(keep, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[b, h] = p @ vc
    return out


def full_attention(q, k, v, scale: Optional[float] = None,
                   rows: Optional[Sequence[int]] = None):
    """Textbook softmax(alpha Q K^T) V per (batch, head), fp64.

    ``rows`` restricts the query rows computed (output [B, H, len(rows), D]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n, D = q.shape
    alpha = 1.0 / math.sqrt(D) if scale is None else float(scale)
    sel = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((B, H, len(sel), D))
    for b in range(B):
        for h in range(H):
            out[b, h] = _softmax_attend(q[b, h][sel], k[b, h], v[b, h], alpha)
    return out


# ---------------------------------------------------------------------------
# Work model (BASA discussion reply, complexity paragraph: O(n^2) against
# O(n*m); the memory keys add G keys per query).
# ---------------------------------------------------------------------------
def window_flops(batch, heads, n, m, G, D) -> int:
    """Multiply-adds x2 of Q K^T and P V over the window and memory keys."""
    return 4 * batch * heads * n * (m + G) * D


def dense_flops(batch, heads, n, D) -> int:
    return 4 * batch * heads * n * n * D


def theoretical_speedup(n: int, m: int, G: int = 0) -> float:
    """Dense flops over window flops: n/m without memory, n/(m+G) with it."""
    return n / (m + G)
