"""CPU model of the LDS schedule of the window-key dK/dV kernel that walks
windows (bwd_dkdv_res_kernel: 8-wave workgroups, one per CU, each taking
every S-th (batch, head, window) unit of its XCD's range), checked over many
interleavings of its waves.

Each wave is a program of steps that mirrors the kernel: the prologue of the
first unit, then per unit the wait for its own loads, its lse / Dv store,
the unit's barrier, its rows of the next unit's token table, pass 0 (dV)
over the query tiles, the dV epilogue, pass 1 (dK) with the count after
each tile (the wave whose count completes the tile loads the next unit's
tile into that buffer; the last tile after the dK epilogue), and its loads
of the next unit's K / V rows, lse and Dv.  The resources:

* tile buffer it, in 8 parts (one wave's share of the tile's loads each);
  a load into it is in flight from its issue until the issuing wave's next
  wait, and may write at any moment of that stretch;
* the lse / Dv arrays in two slots (unit parity), one part per wave;
* the token tables in two slots, row r owned by the wave that writes it;
* one finish count per buffer, never reset.

Every read must find the content the program means -- (unit, tile), or the
unit -- written before it and with no load into it in flight.  The
schedulers interleave the waves at random, in order, in reverse, and with
one wave starved for as long as another can run, so a read that only an
unordered write could satisfy fails.  Planted mistakes (a tile loaded by its
first finisher, one slot for both parities, no wait at the top of a unit,
the table rows shared between waves as a thread-per-row build would) must
each fail.  A last test checks the walk itself: every unit taken by exactly
one workgroup.
"""
import random

import pytest

NW = 8          # waves per workgroup, 32 keys each
KQ = 64         # queries per tile


class Violation(AssertionError):
    pass


def wave_program(w, nit, J, m, mistakes=()):
    """The steps of wave w over J units of a window of m tokens (nit tiles)."""
    one_slot = "one_slot" in mistakes
    slot = (lambda j: 0) if one_slot else (lambda j: j & 1)
    last_wave = 0 if "first_finisher" in mistakes else NW - 1
    keys = [r for r in range(w * 32, w * 32 + 32) if r < m]
    if "shared_rows" in mistakes:
        # rows written by thread r (wave r // 64), read by wave r // 32
        built = [r for r in range(m) if r // 64 == w]
    else:
        built = keys
    kcl = sorted({min(k, m - 1) for k in range(w * 32, w * 32 + 32)})

    def tile_rows(it):
        return sorted({min(it * KQ + r, m - 1) for r in range(KQ)})

    def load_tile(it, j, parts):
        # the token table rows the loads read, then the loads themselves
        for r in tile_rows(it):
            yield ("read", ("tab", slot(j), r), j)
        for part in parts:
            yield ("load", ("buf", it, part), (j, it))

    # prologue: unit 0's rows of the table, the barrier, unit 0's loads
    for r in built:
        yield ("write", ("tab", slot(0), r), 0)
    yield ("barrier",)
    for it in range(nit):
        yield from load_tile(it, 0, [w])
    for r in keys:                                  # K / V rows, lse, Dv
        yield ("read", ("tab", slot(0), r), 0)
    for j in range(J):
        has_next = j + 1 < J
        if "no_wait" not in mistakes:
            yield ("wait",)
        yield ("write", ("lse", slot(j), w), j)
        yield ("barrier",)
        if has_next:
            for r in built:
                yield ("write", ("tab", slot(j + 1), r), j + 1)
        for it in range(nit):                       # pass 0
            for part in range(NW):
                yield ("read", ("buf", it, part), (j, it))
            for part in (2 * it, 2 * it + 1):
                yield ("read", ("lse", slot(j), part), j)
        for r in kcl:                               # dV epilogue
            yield ("read", ("tab", slot(j), r), j)
        last_tile = False
        for it in range(nit):                       # pass 1
            for part in range(NW):
                yield ("read", ("buf", it, part), (j, it))
            for part in (2 * it, 2 * it + 1):
                yield ("read", ("lse", slot(j), part), j)
            if has_next:
                old = yield ("count", it)
                if old % NW == last_wave:
                    if it + 1 < nit:
                        yield from load_tile(it, j + 1, range(NW))
                    else:
                        last_tile = True
        for r in kcl:                               # dK epilogue
            yield ("read", ("tab", slot(j), r), j)
        if last_tile:
            yield from load_tile(nit - 1, j + 1, range(NW))
        if has_next:
            rows = keys if "shared_rows" not in mistakes else [
                r for r in range(m) if r // 32 == w]
            for r in rows:
                yield ("read", ("tab", slot(j + 1), r), j + 1)


def run(nit, J, m, policy, seed=0, mistakes=()):
    rng = random.Random(seed)
    progs = [wave_program(w, nit, J, m, mistakes) for w in range(NW)]
    state = {}            # resource -> content
    flight = {}           # resource -> issuing wave of a load in flight
    queue = [[] for _ in range(NW)]
    cnt = [0] * 4
    pending = [None] * NW  # next step of each wave
    reply = [None] * NW
    at_barrier = [False] * NW
    done = [False] * NW

    def advance(w):
        try:
            pending[w] = progs[w].send(reply[w]) if pending[w] is not None else next(progs[w])
        except StopIteration:
            done[w] = True
            pending[w] = None
        reply[w] = None

    for w in range(NW):
        advance(w)
    starved = rng.randrange(NW)
    while not all(done):
        runnable = [w for w in range(NW) if not done[w] and not at_barrier[w]]
        if not runnable:
            waiting = [w for w in range(NW) if at_barrier[w]]
            if len(waiting) + sum(done) != NW or sum(done):
                raise Violation("a barrier that not every wave reaches")
            for w in waiting:
                at_barrier[w] = False
                advance(w)
            continue
        if policy == "random":
            w = rng.choice(runnable)
        elif policy == "in_order":
            w = runnable[0]
        elif policy == "reverse":
            w = runnable[-1]
        else:   # starve one wave
            others = [x for x in runnable if x != starved]
            w = rng.choice(others) if others else runnable[0]
        step = pending[w]
        kind = step[0]
        if kind == "barrier":
            at_barrier[w] = True
            continue
        if kind == "write":
            res, content = step[1], step[2]
            if res in flight:
                raise Violation(f"wave {w} writes {res} under a load in flight")
            state[res] = content
        elif kind == "read":
            res, want = step[1], step[2]
            if res in flight:
                raise Violation(f"wave {w} reads {res} while a load into it is in flight")
            if state.get(res) != want:
                raise Violation(f"wave {w} reads {res}: holds {state.get(res)}, wants {want}")
        elif kind == "load":
            res, content = step[1], step[2]
            if res in flight:
                raise Violation(f"wave {w} loads into {res} while a load into it is in flight")
            flight[res] = w
            queue[w].append((res, content))
        elif kind == "wait":
            for res, content in queue[w]:
                del flight[res]
                state[res] = content
            queue[w] = []
        elif kind == "count":
            reply[w] = cnt[step[1]]
            cnt[step[1]] += 1
        advance(w)
    if flight:
        raise Violation(f"loads in flight at the end: {sorted(flight)}")


POLICIES = ("random", "in_order", "reverse", "starve")
SHAPES = [
    # window tokens m (nit = ceil(m / 64) tiles), units per workgroup J
    (129, 1), (129, 3), (169, 2), (192, 2), (225, 3), (256, 1), (256, 2), (256, 6),
]


@pytest.mark.parametrize("m,J", SHAPES)
def test_walk_is_race_free(m, J):
    nit = (m + KQ - 1) // KQ
    for policy in POLICIES:
        for seed in range(40 if policy in ("random", "starve") else 1):
            run(nit, J, m, policy, seed)


@pytest.mark.parametrize("mistake", ["first_finisher", "one_slot", "no_wait", "shared_rows"])
def test_model_catches_planted_mistakes(mistake):
    caught = 0
    for m, J in SHAPES:
        if J < 2:
            continue
        nit = (m + KQ - 1) // KQ
        for policy in POLICIES:
            for seed in range(40):
                try:
                    run(nit, J, m, policy, seed, mistakes=(mistake,))
                except Violation:
                    caught += 1
                    break
    assert caught > 0, mistake


def walk(units, wgs_per_xcd_cap=32):
    """The launch and unit walk of the kernel: grid 8 * min(upx, 32); the
    workgroup at blockIdx b takes first = (b % 8) * upx + b // 8 and every
    (grid / 8)-th unit after it below the end of its XCD's range."""
    upx = (units + 7) // 8
    per_xcd = min(upx, wgs_per_xcd_cap)
    grid = 8 * per_xcd
    S = grid // 8
    taken = []
    for b in range(grid):
        ubeg = (b & 7) * upx
        uend = min(ubeg + upx, units)
        first = ubeg + (b >> 3)
        if first >= uend:
            continue
        J = (uend - first + S - 1) // S
        us = [first + j * S for j in range(J)]
        assert all(u < uend for u in us)
        taken += us
    return taken


@pytest.mark.parametrize("units", [1, 7, 8, 9, 100, 255, 256, 257, 432, 576, 1536, 1537, 98304])
def test_walk_takes_every_unit_once(units):
    taken = walk(units)
    assert sorted(taken) == list(range(units))
