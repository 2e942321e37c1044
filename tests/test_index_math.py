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
* The output rows of the persistent kernel pass through each wave's staging
  area (attn_bf16.hip: finish_lds): the writes from the accumulator layout
  and the reads back for whole-row stores must be inverse maps of every
  (row, 16-byte chunk).
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


def _staged_output_maps(D):
    """The persistent kernel's output path (finish_lds): lane (l32, hf) holds,
    for d block db and group pair g in {0, 2}, the 8 d values of chunk
    c = 4 db + g + 1 - hf of query row l32 after the lane-pair exchange, and
    writes them to staging byte (l32 * CPR + (c ^ (l32 % CPR))) * 16.  Store
    instruction i then reads byte i * 1024 + 16 * lane and writes it to row
    r = (64 / CPR) i + lane / CPR at byte 16 * ((lane % CPR) ^ (r % CPR))."""
    CPR, DB = D // 8, D // 32
    writes = {}
    for l32 in range(32):
        for hf in range(2):
            for db in range(DB):
                for g in (0, 2):
                    c = db * 4 + g + 1 - hf
                    slot = l32 * CPR + (c ^ (l32 % CPR))
                    assert slot not in writes
                    writes[slot] = (l32, c)
    reads = {}
    for i in range(32 * CPR // 64):
        for lane in range(64):
            r = (64 // CPR) * i + lane // CPR
            ch = (lane % CPR) ^ (r % CPR)
            slot = (i * 1024 + lane * 16) // 16
            reads[slot] = (r, ch)
    return CPR, writes, reads


def test_staged_output_transpose_is_exact():
    for D in (64, 128):
        CPR, writes, reads = _staged_output_maps(D)
        # every (row, chunk) of the wave's 32 rows written once, read back once,
        # and stored at its own row and chunk
        assert sorted(writes.values()) == [(r, c) for r in range(32) for c in range(CPR)]
        assert set(writes) == set(reads)
        for slot, rc in reads.items():
            assert writes[slot] == rc, (D, slot)


def test_staged_output_writes_spread_over_banks():
    # a b128 LDS access is served 16 lanes at a time; the 16 lanes of each
    # quarter wave should land in distinct 16-byte slots modulo 256 bytes (the
    # 64 banks of 4 bytes).  At D = 128 (one row per 256 bytes) the writes do;
    # at D = 64 rows r and r + 8 share a slot (2-way, on the four writes per
    # wave and unit).  The reads back are contiguous.
    for D, distinct in ((64, 8), (128, 16)):
        CPR, DB = D // 8, D // 32
        for hf in range(2):
            for db in range(DB):
                for g in (0, 2):
                    c = db * 4 + g + 1 - hf
                    for q0 in range(0, 32, 16):
                        banks = [((l32 * CPR + (c ^ (l32 % CPR))) * 16 // 16) % 16
                                 for l32 in range(q0, q0 + 16)]
                        assert len(set(banks)) == distinct, (D, hf, db, g, q0)
        for i in range(32 * CPR // 64):
            for q in range(4):
                banks = [((i * 1024 + lane * 16) // 16) % 16 for lane in range(16 * q, 16 * q + 16)]
                assert len(set(banks)) == 16
