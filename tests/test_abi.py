"""C ABI checks that need no GPU.

The library loads, exports every function include/basa.h declares, its
host-only helpers give the right values, and every argument error is
reported before anything is enqueued (the fake device pointers used here are
never dereferenced: validation returns first).
"""
import ctypes
import json
import os
import re

import pytest

import sparse_window_attention_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "basa.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced
SZ = 1 << 30           # spacing between fake buffers (no false overlaps)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(basa_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 18, names
    lib = ctypes.CDLL(S.library_path)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in (0, 1, 2, 3):
        assert S.lib.basa_status_string(code).decode().startswith("BASA_")
    assert S.lib.basa_status_string(99).decode() == "unknown status"
    assert S.version() >= 100


def test_shift_helper_matches_workload_text():
    cases = json.load(open(os.path.join(GOLDEN, "shift_schedules.json")))["cases"]
    for c in cases:
        for b, want in enumerate(c["shifts"]):
            assert list(S.shift_for_block(b, c["schedule"], c["window"])) == want, c["name"]
    got = [S.shift_for_block(b, S.SCHED_FOUR_PHASE, (7, 10, 13)) for b in range(8)]
    assert got == [(0, 0, 0), (3, 0, 0), (0, 5, 0), (3, 5, 0), (0, 0, 6), (3, 0, 6),
                   (0, 5, 6), (3, 5, 6)]


def test_shift_helper_errors():
    for args in [(-1, 1, (2, 2)), (0, 7, (2, 2)), (0, 1, (0, 2))]:
        with pytest.raises(S.BasaError) as e:
            S.shift_for_block(*args)
        assert e.value.status == S.BASA_ERR_INVALID_ARG
    out = (ctypes.c_int32 * 4)()
    assert S.lib.basa_shift_for_block(0, 1, 4, S._arr([2, 2, 2, 2]), out) == S.BASA_ERR_INVALID_ARG
    assert S.lib.basa_shift_for_block(0, 1, 2, None, out) == S.BASA_ERR_INVALID_ARG


def test_mem_tokens():
    assert S.mem_tokens((64, 64), (4, 4)) == 256
    assert S.mem_tokens((128, 128), (8, 8)) == 256
    assert S.mem_tokens((21, 30, 52), (3, 5, 4)) == 546
    assert S.mem_tokens((21, 30, 52), (1, 5, 4)) == 1638
    assert S.mem_tokens((512, 512), (8, 8)) == 4096
    for g, p in [((4, 6), (3, 3)), ((4, 6), (0, 3)), ((0, 6), (1, 3))]:
        assert S.lib.basa_mem_tokens(2, S._arr(g), S._arr(p)) == -1
    assert S.lib.basa_mem_tokens(4, S._arr((1, 2, 3, 4)), S._arr((1, 1, 1, 1))) == -1


def _win(**kw):
    a = dict(q=FAKE, k=FAKE + SZ, v=FAKE + 2 * SZ, km=None, vm=None, G=0, out=FAKE + 3 * SZ,
             B=1, H=2, D=128, grid=(8, 8), window=(4, 4), shift=(0, 0), scale=-1.0, bias=0.0,
             dtype=S.BASA_BF16, layout=S.BASA_LAYOUT_BHND)
    a.update(kw)
    nd = len(a["grid"])
    return S.lib.basa_window_attn(
        a["q"], a["k"], a["v"], a["km"], a["vm"], a["G"], a["out"], a["B"], a["H"], a["D"],
        a.get("ndim", nd), S._arr(a["grid"]), S._arr(a["window"]), S._arr(a["shift"]),
        a["scale"], a["bias"], a["dtype"], a["layout"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), S.BASA_ERR_INVALID_ARG),
    (dict(out=None), S.BASA_ERR_INVALID_ARG),
    (dict(ndim=4, grid=(8, 8, 8, 8), window=(4, 4, 4, 4), shift=(0, 0, 0, 0)), S.BASA_ERR_INVALID_ARG),
    (dict(ndim=1, grid=(8,), window=(4,), shift=(0,)), S.BASA_ERR_INVALID_ARG),
    (dict(grid=(8, 0)), S.BASA_ERR_INVALID_ARG),
    (dict(window=(3, 4)), S.BASA_ERR_INVALID_ARG),
    (dict(window=(0, 4)), S.BASA_ERR_INVALID_ARG),
    (dict(km=FAKE + 4 * SZ), S.BASA_ERR_INVALID_ARG),               # k_mem without v_mem
    (dict(km=FAKE + 4 * SZ, vm=FAKE + 5 * SZ, G=0), S.BASA_ERR_INVALID_ARG),
    (dict(G=4), S.BASA_ERR_INVALID_ARG),                            # n_mem without memory
    (dict(out=FAKE + 64), S.BASA_ERR_INVALID_ARG),                  # out overlaps q
    (dict(km=FAKE + 4 * SZ, vm=FAKE + 3 * SZ + 256, G=4), S.BASA_ERR_INVALID_ARG),  # out overlaps v_mem
    (dict(q=FAKE + 8), S.BASA_ERR_INVALID_ARG),                     # misaligned
    (dict(B=-1), S.BASA_ERR_INVALID_ARG),
    (dict(layout=5), S.BASA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), S.BASA_ERR_INVALID_ARG),
    (dict(bias=float("inf")), S.BASA_ERR_INVALID_ARG),
    (dict(D=96), S.BASA_ERR_UNSUPPORTED),
    (dict(dtype=7), S.BASA_ERR_UNSUPPORTED),
    (dict(grid=(128, 128), window=(128, 64)), S.BASA_ERR_UNSUPPORTED),  # 8192-token window
])
def test_window_attn_validation(kw, code):
    assert _win(**kw) == code
    assert len(S.lib.basa_last_error().decode()) > 5


def test_pool_validation():
    f = S.lib.basa_pool_kv
    args = lambda **kw: dict(dict(k=FAKE, v=FAKE + SZ, km=FAKE + 2 * SZ, vm=FAKE + 3 * SZ, B=1,
                                  H=1, D=64, grid=(8, 8), pool=(4, 4), dtype=S.BASA_BF16,
                                  layout=0), **kw)

    def call(a):
        return f(a["k"], a["v"], a["km"], a["vm"], a["B"], a["H"], a["D"], len(a["grid"]),
                 S._arr(a["grid"]), S._arr(a["pool"]), a["dtype"], a["layout"], None)

    assert call(args(k=None)) == S.BASA_ERR_INVALID_ARG
    assert call(args(pool=(3, 4))) == S.BASA_ERR_INVALID_ARG
    assert call(args(km=FAKE + 64)) == S.BASA_ERR_INVALID_ARG      # k_mem inside k
    assert call(args(vm=FAKE + 2 * SZ + 16)) == S.BASA_ERR_INVALID_ARG  # k_mem/v_mem overlap
    assert call(args(D=32)) == S.BASA_ERR_UNSUPPORTED
    assert call(args(dtype=3)) == S.BASA_ERR_UNSUPPORTED


def test_full_attn_validation():
    f = S.lib.basa_full_attn
    assert f(FAKE, FAKE + SZ, FAKE + 2 * SZ, FAKE + 3 * SZ, 1, 1, 0, 64, -1.0, 1, 0, None) \
        == S.BASA_ERR_INVALID_ARG
    assert f(FAKE, FAKE + SZ, FAKE + 2 * SZ, FAKE + 16, 1, 1, 64, 64, -1.0, 1, 0, None) \
        == S.BASA_ERR_INVALID_ARG
    assert f(FAKE, FAKE + SZ, FAKE + 2 * SZ, FAKE + 3 * SZ, 1, 1, 64, 80, -1.0, 1, 0, None) \
        == S.BASA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE + SZ, FAKE + 2 * SZ, FAKE + 3 * SZ, 1, 1, 1 << 26, 128, -1.0, 1, 0,
             None) == S.BASA_ERR_UNSUPPORTED


def test_dense_attn_validation():
    f = S.lib.basa_dense_attn
    q, k, v, o = FAKE, FAKE + SZ, FAKE + 2 * SZ, FAKE + 3 * SZ
    for nq, nkv in ((0, 64), (64, 0), (-1, 64)):
        assert f(q, k, v, o, 1, 2, nq, nkv, 128, -1.0, 1, 0, None) == S.BASA_ERR_INVALID_ARG
    assert f(None, k, v, o, 1, 2, 64, 64, 128, -1.0, 1, 0, None) == S.BASA_ERR_INVALID_ARG
    # out overlapping k, whose extent (n_kv rows) is larger than q's
    assert f(q, k, v, k + 256 * 128 * 2, 1, 1, 16, 512, 128, -1.0, 1, 0, None) \
        == S.BASA_ERR_INVALID_ARG
    assert f(q, k, v, o, 1, 1, 64, 64, 96, -1.0, 1, 0, None) == S.BASA_ERR_UNSUPPORTED
    assert f(q, k, v, o, 1, 1, 64, 1 << 26, 128, -1.0, 1, 0, None) == S.BASA_ERR_UNSUPPORTED
    assert f(q, k, v, o, 1, 1, 64, 64, 128, float("nan"), 1, 0, None) == S.BASA_ERR_INVALID_ARG
    assert f(None, None, None, None, 0, 3, 64, 32, 128, -1.0, 1, 0, None) == S.BASA_OK


def test_center_region_validation():
    out = (ctypes.c_int32 * 16)()
    f = S.lib.basa_center_region
    assert f(8, 8, 2, 2, out) == S.BASA_OK and list(out[:4]) == [27, 28, 35, 36]
    for args in ((8, 8, 0, 2), (8, 8, 9, 2), (8, 8, 2, 9), (0, 8, 1, 1), (8, -1, 1, 1)):
        assert f(*args, out) == S.BASA_ERR_INVALID_ARG, args
    assert f(8, 8, 2, 2, None) == S.BASA_ERR_INVALID_ARG
    assert f(1 << 16, 1 << 16, 1, 1, out) == S.BASA_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        S.center_region_tokens((8, 8, 8), (2, 2))


@pytest.mark.parametrize("call", ["mem_tokens", "pool_kv", "window_attn", "window_attn_fwd",
                                  "window_attn_bwd", "bwd_workspace_bytes"])
def test_binding_checks_geometry_lengths(call):
    # the C side reads ndim = len(grid) entries of every geometry array: a
    # shorter list would be read past its end, a longer one truncated, so the
    # binding refuses both before any tensor is looked at
    x = object()
    grid3 = (21, 30, 52)
    cases = {
        "mem_tokens": [lambda: S.mem_tokens(grid3, (3, 5)),
                       lambda: S.mem_tokens((8, 8), (4, 4, 1))],
        "pool_kv": [lambda: S.pool_kv(x, x, grid3, (3, 5))],
        "window_attn": [lambda: S.window_attn(x, x, x, grid3, (7, 10, 13), (3, 5)),
                        lambda: S.window_attn(x, x, x, grid3, (7, 10), (3, 5, 6)),
                        lambda: S.window_attn(x, x, x, (8, 8), (4, 4), (1, 1, 1)),
                        lambda: S.window_attn(x, x, x, (2, 2, 2, 2), (1, 1, 1, 1), (0, 0, 0, 0))],
        "window_attn_fwd": [lambda: S.window_attn_fwd(x, x, x, grid3, (7, 10, 13), (3, 5))],
        "window_attn_bwd": [lambda: S.window_attn_bwd(x, x, x, x, x, x, grid3, (7, 10, 13),
                                                      (3, 5, 6), pool=(3, 5))],
        "bwd_workspace_bytes": [lambda: S.bwd_workspace_bytes(1, 1, 128, grid3, (3, 5))],
    }
    for fn in cases[call]:
        with pytest.raises(ValueError):
            fn()


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 16, 64)
    with pytest.raises(ValueError):
        S.window_attn(x, x, x, (4, 4), (2, 2), (0, 0))
    with pytest.raises(ValueError):
        S.full_attn(x, x, x)


def test_single_hip_runtime_in_process():
    """The library binds to the HIP runtime torch loaded, whatever the import order."""
    import subprocess
    import sys
    code = ("import sparse_window_attention_amd, torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "1"


def _bwd(**kw):
    a = dict(q=FAKE, k=FAKE + SZ, v=FAKE + 2 * SZ, km=FAKE + 3 * SZ, vm=FAKE + 4 * SZ,
             out=FAKE + 5 * SZ, dout=FAKE + 6 * SZ, lse=FAKE + 7 * SZ, dq=FAKE + 8 * SZ,
             dk=FAKE + 9 * SZ, dv=FAKE + 10 * SZ, ws=FAKE + 11 * SZ, wsb=1 << 28, B=1, H=2,
             D=128, grid=(8, 8), window=(4, 4), shift=(0, 0), pool=(4, 4), scale=-1.0,
             bias=0.0, dtype=S.BASA_BF16, layout=S.BASA_LAYOUT_BHND)
    a.update(kw)
    arr = lambda x: None if x is None else (ctypes.c_int32 * len(x))(*x)
    return S.lib.basa_window_attn_bwd(
        a["q"], a["k"], a["v"], a["km"], a["vm"], a["out"], a["dout"], a["lse"], a["dq"],
        a["dk"], a["dv"], a["ws"], a["wsb"], a["B"], a["H"], a["D"], len(a["grid"]),
        arr(a["grid"]), arr(a["window"]), arr(a["shift"]), arr(a["pool"]), a["scale"],
        a["bias"], a["dtype"], a["layout"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), S.BASA_ERR_INVALID_ARG),
    (dict(lse=None), S.BASA_ERR_INVALID_ARG),
    (dict(ws=None), S.BASA_ERR_INVALID_ARG),
    (dict(pool=None), S.BASA_ERR_INVALID_ARG),                    # memory without pool
    (dict(km=None, vm=None), S.BASA_ERR_INVALID_ARG),             # pool without memory
    (dict(pool=(3, 4)), S.BASA_ERR_INVALID_ARG),                  # pool does not divide
    (dict(window=(3, 4)), S.BASA_ERR_INVALID_ARG),
    (dict(wsb=1024), S.BASA_ERR_INVALID_ARG),                     # workspace too small
    (dict(dq=FAKE + 64), S.BASA_ERR_INVALID_ARG),                 # dq overlaps q
    (dict(dk=FAKE + 8 * SZ + 128), S.BASA_ERR_INVALID_ARG),       # dk overlaps dq
    (dict(ws=FAKE + 7 * SZ), S.BASA_ERR_INVALID_ARG),             # workspace overlaps lse
    (dict(lse=FAKE + 7 * SZ + 2), S.BASA_ERR_INVALID_ARG),        # misaligned lse
    (dict(dtype=S.BASA_F32), S.BASA_ERR_UNSUPPORTED),
    (dict(D=96), S.BASA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), S.BASA_ERR_INVALID_ARG),
])
def test_backward_validation(kw, code):
    assert _bwd(**kw) == code
    assert len(S.lib.basa_last_error().decode()) > 5


def _bwd_noalloc(space=SZ, **kw):
    a = dict(q=FAKE, k=FAKE + space, v=FAKE + 2 * space, km=FAKE + 3 * space,
             vm=FAKE + 4 * space, out=FAKE + 5 * space, dout=FAKE + 6 * space,
             lse=FAKE + 7 * space, dq=FAKE + 8 * space, dk=FAKE + 9 * space,
             dv=FAKE + 10 * space, B=1, H=2, D=128, grid=(8, 8), window=(4, 4), shift=(0, 0),
             pool=(4, 4), scale=-1.0, bias=0.0, dtype=S.BASA_BF16, layout=S.BASA_LAYOUT_BHND)
    a.update(kw)
    arr = lambda x: None if x is None else (ctypes.c_int32 * len(x))(*x)
    return S.lib.basa_window_attn_bwd_noalloc(
        a["q"], a["k"], a["v"], a["km"], a["vm"], a["out"], a["dout"], a["lse"], a["dq"],
        a["dk"], a["dv"], a["B"], a["H"], a["D"], len(a["grid"]), arr(a["grid"]),
        arr(a["window"]), arr(a["shift"]), arr(a["pool"]), a["scale"], a["bias"], a["dtype"],
        a["layout"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), S.BASA_ERR_INVALID_ARG),
    (dict(pool=None), S.BASA_ERR_INVALID_ARG),
    (dict(window=(3, 4)), S.BASA_ERR_INVALID_ARG),
    (dict(dq=FAKE + 64), S.BASA_ERR_INVALID_ARG),
    (dict(dtype=S.BASA_F32), S.BASA_ERR_UNSUPPORTED),
])
def test_noalloc_backward_validation(kw, code):
    # argument errors are reported before the scratch array is looked up
    assert _bwd_noalloc(**kw) == code


def test_noalloc_backward_rejects_workspace_beyond_scratch():
    # 24 heads of the 512 x 512 grid with 4096 memory tokens: even one query
    # chunk per head needs 25 MB of row sums and 2 x 50 MB of memory sums,
    # more than the scratch array; rejected before any HIP call
    big = 1 << 34
    rc = _bwd_noalloc(space=big, H=24, grid=(512, 512), window=(32, 32), pool=(8, 8))
    assert rc == S.BASA_ERR_UNSUPPORTED
    msg = S.lib.basa_last_error().decode()
    assert "scratch" in msg and str(64 << 20) in msg


def test_backward_workspace_size():
    f = S.lib.basa_window_attn_bwd_workspace
    arr = lambda x: (ctypes.c_int32 * len(x))(*x)
    no_mem = f(1, 24, 128, 2, arr((128, 128)), None)
    with_mem = f(1, 24, 128, 2, arr((128, 128)), arr((8, 8)))
    assert no_mem >= 24 * 16384 * 4                     # one fp32 per token
    # memory partials: two fp32 [B*H, chunks of 1024 queries, G, D] and their sums
    assert with_mem >= no_mem + 2 * 24 * 16 * 256 * 128 * 4 + 2 * 24 * 256 * 128 * 4
    assert f(1, 24, 128, 2, arr((128, 128)), arr((3, 8))) == -1
    assert f(1, 24, 96, 2, arr((128, 128)), None) == -1


def test_fwd_lse_validation():
    f = S.lib.basa_window_attn_fwd
    arr = lambda x: (ctypes.c_int32 * len(x))(*x)
    args = [FAKE, FAKE + SZ, FAKE + 2 * SZ, None, None, 0, FAKE + 3 * SZ]
    rest = [1, 2, 128, 2, arr((8, 8)), arr((4, 4)), arr((0, 0)), -1.0, 0.0]
    assert f(*args, None, *rest, S.BASA_BF16, 0, None) == S.BASA_ERR_INVALID_ARG
    assert f(*args, FAKE + 4 * SZ, *rest, S.BASA_F32, 0, None) == S.BASA_ERR_UNSUPPORTED
    assert f(*args, FAKE + 3 * SZ + 64, *rest, S.BASA_BF16, 0, None) == S.BASA_ERR_INVALID_ARG


def test_hilbert_order_validation():
    buf = (ctypes.c_int32 * 16)()
    assert S.lib.basa_hilbert_order(4, buf) == S.BASA_OK
    assert S.lib.basa_hilbert_order(4, None) == S.BASA_ERR_INVALID_ARG
    for side in (0, 3, 6, 1 << 16):
        assert S.lib.basa_hilbert_order(side, buf) == S.BASA_ERR_INVALID_ARG


def _curve(**kw):
    a = dict(q=FAKE, k=FAKE + SZ, v=FAKE + 2 * SZ, km=FAKE + 3 * SZ, vm=FAKE + 4 * SZ, G=64,
             out=FAKE + 5 * SZ, B=1, H=2, D=128, n=4096, order=FAKE + 6 * SZ, tile=256,
             slide=0, scale=-1.0, bias=0.0, dtype=S.BASA_BF16, layout=S.BASA_LAYOUT_BHND)
    a.update(kw)
    return S.lib.basa_curve_attn(a["q"], a["k"], a["v"], a["km"], a["vm"], a["G"], a["out"],
                                 a["B"], a["H"], a["D"], a["n"], a["order"], a["tile"],
                                 a["slide"], a["scale"], a["bias"], a["dtype"], a["layout"],
                                 None)


@pytest.mark.parametrize("kw,code", [
    (dict(order=None), S.BASA_ERR_INVALID_ARG),
    (dict(q=None), S.BASA_ERR_INVALID_ARG),
    (dict(tile=0), S.BASA_ERR_INVALID_ARG),
    (dict(tile=300), S.BASA_ERR_INVALID_ARG),                     # does not divide n
    (dict(n=1 << 14, tile=8192), S.BASA_ERR_UNSUPPORTED),         # tile above the maximum
    (dict(km=None), S.BASA_ERR_INVALID_ARG),                      # one memory operand
    (dict(km=None, vm=None), S.BASA_ERR_INVALID_ARG),             # n_mem without memory
    (dict(G=0), S.BASA_ERR_INVALID_ARG),
    (dict(order=FAKE + 6 * SZ + 2), S.BASA_ERR_INVALID_ARG),      # misaligned order
    (dict(out=FAKE + 6 * SZ), S.BASA_ERR_INVALID_ARG),            # out overlaps order
    (dict(out=FAKE + 64), S.BASA_ERR_INVALID_ARG),                # out overlaps q
    (dict(scale=float("inf")), S.BASA_ERR_INVALID_ARG),
    (dict(bias=float("nan")), S.BASA_ERR_INVALID_ARG),
    (dict(D=96), S.BASA_ERR_UNSUPPORTED),
    (dict(dtype=7), S.BASA_ERR_UNSUPPORTED),
])
def test_curve_attn_validation(kw, code):
    assert _curve(**kw) == code
    assert len(S.lib.basa_last_error().decode()) > 5


@pytest.mark.parametrize("args,code", [
    ((FAKE, FAKE + SZ, None, 64, FAKE + 3 * SZ, FAKE + 4 * SZ), S.BASA_ERR_INVALID_ARG),
    ((FAKE, FAKE + SZ, FAKE + 2 * SZ, 0, FAKE + 3 * SZ, FAKE + 4 * SZ), S.BASA_ERR_INVALID_ARG),
    ((FAKE, FAKE + SZ, FAKE + 2 * SZ + 1, 64, FAKE + 3 * SZ, FAKE + 4 * SZ),
     S.BASA_ERR_INVALID_ARG),
    ((FAKE, FAKE + SZ, FAKE + 2 * SZ, 64, FAKE + 16, FAKE + 4 * SZ), S.BASA_ERR_INVALID_ARG),
    ((FAKE, FAKE + SZ, FAKE + 2 * SZ, 64, FAKE + 3 * SZ, FAKE + 3 * SZ + 64),
     S.BASA_ERR_INVALID_ARG),
])
def test_gather_kv_validation(args, code):
    rc = S.lib.basa_gather_kv(*args, 1, 2, 128, 4096, S.BASA_BF16, S.BASA_LAYOUT_BHND, None)
    assert rc == code
    assert len(S.lib.basa_last_error().decode()) > 5


def test_calib_mfma_validation():
    assert S.lib.basa_calib_mfma(None, 4, 10, None) == S.BASA_ERR_INVALID_ARG
    assert S.lib.basa_calib_mfma(FAKE, 0, 10, None) == S.BASA_ERR_INVALID_ARG
    assert S.lib.basa_calib_mfma(FAKE, 4, 0, None) == S.BASA_ERR_INVALID_ARG


def test_empty_batch_is_a_no_op():
    # batch or heads 0: BASA_OK without reading any pointer (all NULL here),
    # once head_dim, dtype and layout are valid
    arr = S._arr
    for B, H in ((0, 2), (1, 0), (0, 0)):
        assert _win(q=None, k=None, v=None, out=None, B=B, H=H) == S.BASA_OK
        assert S.lib.basa_pool_kv(None, None, None, None, B, H, 128, 2, arr((8, 8)), arr((4, 4)),
                                  S.BASA_BF16, 0, None) == S.BASA_OK
        assert S.lib.basa_full_attn(None, None, None, None, B, H, 64, 128, -1.0, S.BASA_BF16, 0,
                                    None) == S.BASA_OK
        assert S.lib.basa_dense_attn(None, None, None, None, B, H, 64, 96, 128, -1.0, S.BASA_BF16,
                                     0, None) == S.BASA_OK
        assert S.lib.basa_gather_kv(None, None, None, 4, None, None, B, H, 128, 64, S.BASA_BF16, 0,
                                    None) == S.BASA_OK
        assert S.lib.basa_curve_attn(None, None, None, None, None, 0, None, B, H, 128, 64, None, 16,
                                     0, -1.0, 0.0, S.BASA_BF16, 0, None) == S.BASA_OK
        assert _bwd(q=None, k=None, v=None, km=None, vm=None, out=None, dout=None, lse=None,
                    dq=None, dk=None, dv=None, ws=None, B=B, H=H) == S.BASA_OK
    # the scalar arguments are still checked
    assert _win(q=None, k=None, v=None, out=None, B=0, D=96) == S.BASA_ERR_UNSUPPORTED
    assert _win(q=None, k=None, v=None, out=None, B=0, dtype=7) == S.BASA_ERR_UNSUPPORTED
    assert _win(q=None, k=None, v=None, out=None, B=0, layout=3) == S.BASA_ERR_INVALID_ARG
