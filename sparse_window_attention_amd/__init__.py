"""Python binding of the shifted-window sparse attention library (libbasa.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/basa.h``.  torch supplies
device memory and the current stream.  Importing works without a GPU (the
library loads and its host-only helpers run); compute calls need an MI355X.
If ``libbasa.so`` is missing, import fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

__all__ = [
    "BASA_OK", "BASA_ERR_INVALID_ARG", "BASA_ERR_UNSUPPORTED", "BASA_ERR_HIP",
    "BASA_F32", "BASA_BF16", "BASA_LAYOUT_BHND", "BASA_LAYOUT_BNHD",
    "SCHED_NONE", "SCHED_ALTERNATE", "SCHED_FOUR_PHASE", "BasaError", "lib",
    "library_path", "version", "mem_tokens", "shift_for_block", "pool_kv",
    "window_attn", "window_attn_fwd", "window_attn_bwd", "window_attn_bwd_noalloc",
    "bwd_workspace_bytes", "full_attn",
    "dense_attn", "hilbert_order", "center_region_tokens", "gather_kv", "curve_attn",
]

BASA_OK, BASA_ERR_INVALID_ARG, BASA_ERR_UNSUPPORTED, BASA_ERR_HIP = 0, 1, 2, 3
BASA_F32, BASA_BF16 = 0, 1
BASA_LAYOUT_BHND, BASA_LAYOUT_BNHD = 0, 1
SCHED_NONE, SCHED_ALTERNATE, SCHED_FOUR_PHASE = 0, 1, 2
MAX_WINDOW_TOKENS = 4096

# BASA_LIBRARY may point at another build of the same library (tuning runs).
library_path = os.environ.get("BASA_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libbasa.so")


class BasaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime (SONAME libamdhip64.so.7).  Importing
    # torch first makes libbasa.so bind to that same runtime, so device
    # pointers and streams from torch are valid in the library's calls; loading
    # libbasa.so first would pull in a second runtime beside torch's.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is not built; run `python -m sparse_window_attention_amd._build`")
    L = ctypes.CDLL(library_path)
    i32, i64, f32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    pi32 = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "basa_version": (i32, []),
        "basa_status_string": (ctypes.c_char_p, [i32]),
        "basa_last_error": (ctypes.c_char_p, []),
        "basa_mem_tokens": (i64, [i32, pi32, pi32]),
        "basa_shift_for_block": (ctypes.c_int, [i32, i32, i32, pi32, pi32]),
        "basa_pool_kv": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, i32, pi32, pi32,
                                        i32, i32, vp]),
        "basa_window_attn": (ctypes.c_int, [vp, vp, vp, vp, vp, i64, vp, i32, i32, i32,
                                            i32, pi32, pi32, pi32, f32, f32, i32, i32, vp]),
        "basa_full_attn": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i64, i32, f32, i32,
                                          i32, vp]),
        "basa_dense_attn": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i64, i64, i32, f32, i32,
                                           i32, vp]),
        "basa_center_region": (ctypes.c_int, [i32, i32, i32, i32, pi32]),
        "basa_window_attn_fwd": (ctypes.c_int, [vp, vp, vp, vp, vp, i64, vp, vp, i32, i32, i32,
                                                i32, pi32, pi32, pi32, f32, f32, i32, i32, vp]),
        "basa_window_attn_bwd_workspace": (i64, [i32, i32, i32, i32, pi32, pi32]),
        "basa_hilbert_order": (ctypes.c_int, [i32, pi32]),
        "basa_calib_mfma": (ctypes.c_int, [vp, i32, i32, vp]),
        "basa_gather_kv": (ctypes.c_int, [vp, vp, vp, i64, vp, vp, i32, i32, i32, i64, i32, i32,
                                          vp]),
        "basa_curve_attn": (ctypes.c_int, [vp, vp, vp, vp, vp, i64, vp, i32, i32, i32, i64, vp,
                                           i32, i64, f32, f32, i32, i32, vp]),
        "basa_window_attn_bwd": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                i64, i32, i32, i32, i32, pi32, pi32, pi32, pi32,
                                                f32, f32, i32, i32, vp]),
        "basa_window_attn_bwd_noalloc": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                        vp, i32, i32, i32, i32, pi32, pi32, pi32,
                                                        pi32, f32, f32, i32, i32, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


def _arr(vals: Sequence[int]):
    vals = [int(v) for v in vals]
    return (ctypes.c_int32 * len(vals))(*vals)


def _ndim(grid: Sequence[int], **parts) -> int:
    """len(grid) after checking that it is 2 or 3 and that every other
    geometry argument (window, shift, pool; None = absent) has as many
    entries: the C side reads ndim entries from each array."""
    nd = len(grid)
    if nd not in (2, 3):
        raise ValueError(f"grid must have 2 or 3 entries (got {nd})")
    for name, val in parts.items():
        if val is not None and len(val) != nd:
            raise ValueError(f"{name} has {len(val)} entries; the grid has {nd}")
    return nd


def _check(status: int) -> None:
    if status != BASA_OK:
        raise BasaError(status, f"{lib.basa_status_string(status).decode()}: "
                                f"{lib.basa_last_error().decode()}")


def version() -> int:
    return int(lib.basa_version())


def mem_tokens(grid: Sequence[int], pool: Sequence[int]) -> int:
    g = lib.basa_mem_tokens(_ndim(grid, pool=pool), _arr(grid), _arr(pool))
    if g < 0:
        raise BasaError(BASA_ERR_INVALID_ARG, lib.basa_last_error().decode())
    return int(g)


def shift_for_block(block: int, schedule: int, window: Sequence[int]) -> Tuple[int, ...]:
    out = (ctypes.c_int32 * len(window))()
    _check(lib.basa_shift_for_block(int(block), int(schedule), len(window), _arr(window), out))
    return tuple(int(x) for x in out)


# ------------------------------------------------------------ tensor calls
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BASA_BF16
    if t.dtype == torch.float32:
        return BASA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _layout_dims(t, layout: str):
    if t.dim() != 4:
        raise ValueError("tensors must be 4-D")
    if layout == "bhnd":
        B, H, n, D = t.shape
        return B, H, n, D, BASA_LAYOUT_BHND
    if layout == "bnhd":
        B, n, H, D = t.shape
        return B, H, n, D, BASA_LAYOUT_BNHD
    raise ValueError("layout must be 'bhnd' or 'bnhd'")


def _check_tensors(*ts):
    t0 = ts[0]
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU")
        if t.device != t0.device:
            raise ValueError("tensors must share one device")
        if t.dtype != t0.dtype:
            raise ValueError("tensors must share one dtype")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def pool_kv(k, v, grid: Sequence[int], pool: Sequence[int], layout: str = "bhnd",
            out: Optional[tuple] = None):
    """Mean-pooled memory (k_mem, v_mem), each [B, H, G, D]."""
    torch = _torch()
    nd = _ndim(grid, pool=pool)
    _check_tensors(k, v)
    B, H, n, D, lay = _layout_dims(k, layout)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v shapes differ")
    G = mem_tokens(grid, pool)
    if out is None:
        km = torch.empty((B, H, G, D), dtype=k.dtype, device=k.device)
        vm = torch.empty_like(km)
    else:
        km, vm = out
        _check_tensors(k, km, vm)
        if tuple(km.shape) != (B, H, G, D) or tuple(vm.shape) != (B, H, G, D):
            raise ValueError("memory outputs must be [B, H, G, D]")
    if n != math.prod(grid):
        raise ValueError("token count does not match the grid")
    _check(lib.basa_pool_kv(k.data_ptr(), v.data_ptr(), km.data_ptr(), vm.data_ptr(), B, H, D,
                            nd, _arr(grid), _arr(pool), _dtype_code(k), lay, _stream(k)))
    return km, vm


def window_attn(q, k, v, grid: Sequence[int], window: Sequence[int], shift: Sequence[int],
                mem: Optional[tuple] = None, scale: Optional[float] = None,
                mem_bias: float = 0.0, out=None, layout: str = "bhnd"):
    """Shifted local window attention with optional pooled memory (k_mem, v_mem)."""
    torch = _torch()
    nd = _ndim(grid, window=window, shift=shift)
    _check_tensors(q, k, v)
    B, H, n, D, lay = _layout_dims(q, layout)
    if tuple(k.shape) != tuple(q.shape) or tuple(v.shape) != tuple(q.shape):
        raise ValueError("q, k, v shapes differ")
    if n != math.prod(grid):
        raise ValueError("token count does not match the grid")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensors(q, out)
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError("out shape differs from q")
    km_p = vm_p = None
    G = 0
    if mem is not None:
        km, vm = mem
        _check_tensors(q, km, vm)
        if km.dim() != 4 or tuple(km.shape[:2]) != (B, H) or km.shape[3] != D \
                or tuple(vm.shape) != tuple(km.shape):
            raise ValueError("memory tensors must be [B, H, G, D]")
        G = km.shape[2]
        km_p, vm_p = km.data_ptr(), vm.data_ptr()
    s = -1.0 if scale is None else float(scale)
    if scale is not None and not scale > 0:
        raise ValueError("scale must be positive")
    _check(lib.basa_window_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), km_p, vm_p, G,
                                out.data_ptr(), B, H, D, nd, _arr(grid), _arr(window),
                                _arr(shift), s, float(mem_bias), _dtype_code(q), lay,
                                _stream(q)))
    return out


def _mem_args(q, mem, B, H, D):
    if mem is None:
        return None, None, 0
    km, vm = mem
    _check_tensors(q, km, vm)
    if km.dim() != 4 or tuple(km.shape[:2]) != (B, H) or km.shape[3] != D \
            or tuple(vm.shape) != tuple(km.shape):
        raise ValueError("memory tensors must be [B, H, G, D]")
    return km.data_ptr(), vm.data_ptr(), km.shape[2]


def window_attn_fwd(q, k, v, grid: Sequence[int], window: Sequence[int], shift: Sequence[int],
                    mem: Optional[tuple] = None, scale: Optional[float] = None,
                    mem_bias: float = 0.0, out=None, lse=None, layout: str = "bhnd"):
    """window_attn that also returns the per-query log-sum-exp (fp32 [B, H, n])
    the backward needs: returns (out, lse)."""
    torch = _torch()
    nd = _ndim(grid, window=window, shift=shift)
    _check_tensors(q, k, v)
    B, H, n, D, lay = _layout_dims(q, layout)
    if tuple(k.shape) != tuple(q.shape) or tuple(v.shape) != tuple(q.shape):
        raise ValueError("q, k, v shapes differ")
    if n != math.prod(grid):
        raise ValueError("token count does not match the grid")
    out = torch.empty_like(q) if out is None else out
    _check_tensors(q, out)
    if lse is None:
        lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
    elif lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, n) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, n] tensor")
    km_p, vm_p, G = _mem_args(q, mem, B, H, D)
    s = -1.0 if scale is None else float(scale)
    if scale is not None and not scale > 0:
        raise ValueError("scale must be positive")
    _check(lib.basa_window_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), km_p, vm_p, G,
                                    out.data_ptr(), lse.data_ptr(), B, H, D, nd,
                                    _arr(grid), _arr(window), _arr(shift), s, float(mem_bias),
                                    _dtype_code(q), lay, _stream(q)))
    return out, lse


def bwd_workspace_bytes(batch: int, heads: int, head_dim: int, grid: Sequence[int],
                        pool: Optional[Sequence[int]] = None) -> int:
    b = lib.basa_window_attn_bwd_workspace(int(batch), int(heads), int(head_dim),
                                           _ndim(grid, pool=pool),
                                           _arr(grid), None if pool is None else _arr(pool))
    if b < 0:
        raise BasaError(BASA_ERR_INVALID_ARG, "invalid shape for the backward workspace")
    return int(b)


def window_attn_bwd(q, k, v, out, dout, lse, grid: Sequence[int], window: Sequence[int],
                    shift: Sequence[int], mem: Optional[tuple] = None,
                    pool: Optional[Sequence[int]] = None, scale: Optional[float] = None,
                    mem_bias: float = 0.0, grads: Optional[tuple] = None, workspace=None,
                    layout: str = "bhnd"):
    """Gradients (dq, dk, dv) of window_attn; with memory, ``mem`` must be
    pool_kv(k, v, grid, pool) and its gradient is folded into dk and dv."""
    torch = _torch()
    nd = _ndim(grid, window=window, shift=shift, pool=pool)
    _check_tensors(q, k, v, out, dout)
    B, H, n, D, lay = _layout_dims(q, layout)
    for t in (k, v, out, dout):
        if tuple(t.shape) != tuple(q.shape):
            raise ValueError("q, k, v, out, dout shapes differ")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, n) or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, n] tensor on q's device")
    if (mem is None) != (pool is None):
        raise ValueError("mem and pool go together")
    km_p, vm_p, _ = _mem_args(q, mem, B, H, D)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    dq, dk, dv = grads
    _check_tensors(q, dq, dk, dv)
    need = bwd_workspace_bytes(B, H, D, grid, pool)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    s = -1.0 if scale is None else float(scale)
    if scale is not None and not scale > 0:
        raise ValueError("scale must be positive")
    _check(lib.basa_window_attn_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), km_p, vm_p, out.data_ptr(), dout.data_ptr(),
        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), B, H, D, nd, _arr(grid),
        _arr(window), _arr(shift), None if pool is None else _arr(pool), s, float(mem_bias),
        _dtype_code(q), lay, _stream(q)))
    return dq, dk, dv


def window_attn_bwd_noalloc(q, k, v, out, dout, lse, grid: Sequence[int],
                            window: Sequence[int], shift: Sequence[int],
                            mem: Optional[tuple] = None, pool: Optional[Sequence[int]] = None,
                            scale: Optional[float] = None, mem_bias: float = 0.0,
                            grads: Optional[tuple] = None, layout: str = "bhnd"):
    """window_attn_bwd with the library's static per-GPU scratch array as the
    workspace (basa_window_attn_bwd_noalloc): the library allocates nothing.
    ``grads`` (dq, dk, dv) are the caller's outputs; pass them to keep the
    call free of allocations on the torch side as well."""
    torch = _torch()
    nd = _ndim(grid, window=window, shift=shift, pool=pool)
    _check_tensors(q, k, v, out, dout)
    B, H, n, D, lay = _layout_dims(q, layout)
    for t in (k, v, out, dout):
        if tuple(t.shape) != tuple(q.shape):
            raise ValueError("q, k, v, out, dout shapes differ")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, n) or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, n] tensor on q's device")
    if (mem is None) != (pool is None):
        raise ValueError("mem and pool go together")
    km_p, vm_p, _ = _mem_args(q, mem, B, H, D)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    dq, dk, dv = grads
    _check_tensors(q, dq, dk, dv)
    for t in grads:
        if tuple(t.shape) != tuple(q.shape):
            raise ValueError("gradient outputs must have q's shape")
    s = -1.0 if scale is None else float(scale)
    if scale is not None and not scale > 0:
        raise ValueError("scale must be positive")
    _check(lib.basa_window_attn_bwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), km_p, vm_p, out.data_ptr(), dout.data_ptr(),
        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, D, nd, _arr(grid),
        _arr(window), _arr(shift), None if pool is None else _arr(pool), s, float(mem_bias),
        _dtype_code(q), lay, _stream(q)))
    return dq, dk, dv


def calib_mfma(sink, blocks: int, iters: int):
    """Runs the bf16 MFMA calibration loop (blocks x 8 waves x iters x 4
    products of 32768 flops) on the current stream; returns its flop count.
    ``sink`` is a float32 GPU tensor of at least ``blocks`` elements."""
    torch = _torch()
    if sink.dtype != torch.float32 or not sink.is_cuda or sink.numel() < blocks:
        raise ValueError("sink must be a float32 GPU tensor of at least `blocks` elements")
    _check(lib.basa_calib_mfma(sink.data_ptr(), int(blocks), int(iters), _stream(sink)))
    return int(blocks) * 8 * int(iters) * 4 * 32768


def full_attn(q, k, v, scale: Optional[float] = None, out=None, layout: str = "bhnd"):
    """Dense softmax(scale q k^T) v over all tokens of each (batch, head)."""
    torch = _torch()
    _check_tensors(q, k, v)
    B, H, n, D, lay = _layout_dims(q, layout)
    if tuple(k.shape) != tuple(q.shape) or tuple(v.shape) != tuple(q.shape):
        raise ValueError("q, k, v shapes differ")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensors(q, out)
    s = -1.0 if scale is None else float(scale)
    if scale is not None and not scale > 0:
        raise ValueError("scale must be positive")
    _check(lib.basa_full_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, n,
                              D, s, _dtype_code(q), lay, _stream(q)))
    return out


def dense_attn(q, k, v, scale: Optional[float] = None, out=None, layout: str = "bhnd"):
    """Dense softmax(scale q k^T) v with n_q queries and n_kv keys per (batch,
    head): q [B, H, n_q, D], k and v [B, H, n_kv, D] (or the BNHD forms)."""
    torch = _torch()
    _check_tensors(q, k, v)
    B, H, nq, D, lay = _layout_dims(q, layout)
    Bk, Hk, nkv, Dk, _ = _layout_dims(k, layout)
    if (Bk, Hk, Dk) != (B, H, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must share q's batch, heads and head dim, and one shape")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensors(q, out)
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError("out shape differs from q")
    s = -1.0 if scale is None else float(scale)
    if scale is not None and not scale > 0:
        raise ValueError("scale must be positive")
    _check(lib.basa_dense_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H,
                               nq, nkv, D, s, _dtype_code(q), lay, _stream(q)))
    return out


# ------------------------------------------------------- Hilbert-order tiles
def hilbert_order(side: int):
    """Raster token index of every position of the Hilbert curve over a
    side x side grid (host numpy int32 [side*side])."""
    import numpy as np
    out = np.empty(int(side) * int(side), dtype=np.int32)
    _check(lib.basa_hilbert_order(int(side), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return out


def center_region_tokens(grid: Sequence[int], size: Sequence[int]):
    """Raster indices of the size[0] x size[1] block at the centre of a 2-D
    grid (basa_center_region), host numpy int32."""
    import numpy as np
    if len(grid) != 2 or len(size) != 2:
        raise ValueError("grid and size must have 2 entries")
    out = np.empty(int(size[0]) * int(size[1]), dtype=np.int32)
    _check(lib.basa_center_region(int(grid[0]), int(grid[1]), int(size[0]), int(size[1]),
                                  out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return out


def gather_kv(k, v, idx, layout: str = "bhnd", out: Optional[tuple] = None):
    """(k[:, :, idx], v[:, :, idx]) as [B, H, len(idx), D] tensors; idx is an
    int32 tensor on the GPU."""
    torch = _torch()
    _check_tensors(k, v)
    B, H, n, D, lay = _layout_dims(k, layout)
    if idx.dtype != torch.int32 or not idx.is_cuda or not idx.is_contiguous() or idx.dim() != 1:
        raise ValueError("idx must be a contiguous int32 vector on the GPU")
    G = idx.numel()
    if out is None:
        ko = torch.empty((B, H, G, D), dtype=k.dtype, device=k.device)
        vo = torch.empty_like(ko)
    else:
        ko, vo = out
        _check_tensors(k, ko, vo)
        if tuple(ko.shape) != (B, H, G, D) or tuple(vo.shape) != (B, H, G, D):
            raise ValueError(f"gather outputs must have shape {(B, H, G, D)}")
    _check(lib.basa_gather_kv(k.data_ptr(), v.data_ptr(), idx.data_ptr(), G, ko.data_ptr(),
                              vo.data_ptr(), B, H, D, n, _dtype_code(k), lay, _stream(k)))
    return ko, vo


def curve_attn(q, k, v, order, tile: int, slide: int = 0, mem: Optional[tuple] = None,
               scale: Optional[float] = None, mem_bias: float = 0.0, out=None,
               layout: str = "bhnd"):
    """Attention inside tiles of `tile` consecutive positions of a token order
    (int32 tensor [n] on the GPU, e.g. hilbert_order), slid by `slide`
    positions, with optional memory keys (e.g. gather_kv of a shared region)."""
    torch = _torch()
    _check_tensors(q, k, v)
    B, H, n, D, lay = _layout_dims(q, layout)
    if tuple(k.shape) != tuple(q.shape) or tuple(v.shape) != tuple(q.shape):
        raise ValueError("q, k, v shapes differ")
    if order.dtype != torch.int32 or not order.is_cuda or order.numel() != n \
            or not order.is_contiguous():
        raise ValueError("order must be a contiguous int32 [n] tensor on the GPU")
    out = torch.empty_like(q) if out is None else out
    _check_tensors(q, out)
    km_p, vm_p, G = _mem_args(q, mem, B, H, D)
    s = -1.0 if scale is None else float(scale)
    if scale is not None and not scale > 0:
        raise ValueError("scale must be positive")
    _check(lib.basa_curve_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), km_p, vm_p, G,
                               out.data_ptr(), B, H, D, n, order.data_ptr(), int(tile),
                               int(slide), s, float(mem_bias), _dtype_code(q), lay, _stream(q)))
    return out
