"""Integer identities the kernels' index arithmetic relies on, checked over
their whole domains on the CPU (uint32 arithmetic written out as the device
code does it).

* window_token divides a slot index r < 4096 by a window dimension
  d <= 4096 as the high 32 bits of r * (floor((2^32 - 1) / d) + 1)
  (basa_common.h: magic_of, div_magic).
* The optional interleaved key-tile order of the persistent kernel
  (BASA_TILE_INTERLEAVE) maps loop position p < t1 to key tile
  c(p) if c(p+1) > c(p) else nw + p - c(p), with c(p) = ceil(p * nw / t1)
  computed as a multiply by floor((2^32 - 1) / t1) + 1; it must be a
  bijection of [0, t1) that keeps window tiles and other tiles each in
  order, for t1 <= 1024 and nw <= 64.
"""
import numpy as np


def magic_of(d):
    return 0 if d <= 1 else (0xFFFFFFFF // d + 1) & 0xFFFFFFFF


def test_div_magic_exact_for_every_slot_and_window_size():
    x = np.arange(4096, dtype=np.uint64)
    for d in range(1, 4097):
        m = magic_of(d)
        q = x if m == 0 else (x * np.uint64(m)) >> np.uint64(32)
        assert np.array_equal(q, x // np.uint64(d)), d


def _tile_order(t1, nw):
    rcp = (0xFFFFFFFF // max(t1, 1) + 1) & 0xFFFFFFFF
    out = []
    for pos in range(t1):
        if nw >= t1 or nw == 0:
            out.append(pos)
            continue
        c0 = ((pos * nw + t1 - 1) * rcp) >> 32
        c1 = (((pos + 1) * nw + t1 - 1) * rcp) >> 32
        out.append(c0 if c1 > c0 else nw + pos - c0)
    return out


def test_interleaved_tile_order_is_an_ordered_bijection():
    for t1 in list(range(1, 130)) + [255, 256, 511, 777, 1000, 1024]:
        for nw in range(0, min(t1, 64) + 1):
            seq = _tile_order(t1, nw)
            assert sorted(seq) == list(range(t1)), (t1, nw)
            w = [x for x in seq if x < nw]
            o = [x for x in seq if x >= nw]
            assert w == sorted(w) and o == sorted(o), (t1, nw)


def test_interleaved_tile_order_examples():
    # window tiles (W) spread among memory tiles (m): the FLUX-2048 shapes
    show = lambda t1, nw: "".join("W" if k < nw else "m" for k in _tile_order(t1, nw))
    assert show(8, 4) == "WmWmWmWm"            # 16x16 windows, 256 memory tokens
    assert show(20, 16) == "WWWWm" * 4          # 32x32 windows, 256 memory tokens
