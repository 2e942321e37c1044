"""CPU model of the LDS and load schedule of the persistent bf16 attention
kernel (attn_bf16_persistent_kernel, direct tile loads), checked for every
unit walk a workgroup can have.

The model walks the kernel's control flow -- the prologue of the first unit,
the top of each unit, the iterations of the tile loop, the last tile and the
step to the next unit -- and records what each wave does to LDS and to its
queue of vector memory operations:

* a direct tile load (buffer -> LDS) is an operation in the wave's queue; it
  writes its LDS buffer at some time until it completes;
* s_waitcnt vmcnt(N) completes all but the N most recent operations (a
  wave's vector memory operations complete in issue order);
* a barrier publishes the completed loads of every wave (the waves run the
  same program, so one wave's queue stands for all); the stretch between two
  barriers is a segment;
* a read of a tile buffer (score or P V operands) must see the tile the
  program means -- (unit, key tile) -- published by an earlier barrier, with
  no load into that buffer in flight;
* a load into a buffer must come after every read of the buffer's previous
  tile, in a later segment (other waves may still be reading in the same
  segment);
* a wave's own Q staging area and the per-unit token tables follow the same
  rules (the staging area is private to the wave, so its loads need only
  the wave's own wait before the read);
* the output rows of a unit pass through the wave's staging area (written
  and read back by the wave) after the next unit's Q rows have been read
  from it, so no staging load may be in flight into it then;
* no load or table read ever names a unit past the workgroup's last one.

It is the schedule's specification on the CPU; the kernel runs the same
steps on the GPU.  A wrong buffer index, a missing wait or a load issued one
step too early fails here.
"""
import pytest


class Violation(AssertionError):
    pass


class Model:
    def __init__(self, nkt, J, KD, ipw, QI):
        self.nkt, self.J, self.KD, self.ipw, self.QI = nkt, J, KD, ipw, QI
        self.seg = 0
        self.queue = []            # outstanding ops of the wave: (buffer, content)
        self.completed = []        # completed, not yet published
        self.visible = {}          # buffer -> published content
        self.pending = {}          # buffer -> content of a load in flight or unpublished
        self.last_read = {}        # buffer -> segment of the last read of its content
        self.reads = []            # (kind, content) in order

    # -- primitives
    def issue(self, buf, content, n=1):
        if content[1] >= self.J:
            raise Violation(f"load for unit {content[1]} past the last unit ({self.J - 1})")
        if buf in self.pending:
            raise Violation(f"load into {buf} while a load into it is in flight")
        if self.last_read.get(buf, -1) >= self.seg:
            raise Violation(f"load into {buf} in the segment where its tile is read")
        self.pending[buf] = content
        for _ in range(n):
            self.queue.append((buf, content))

    def store(self, n=1):
        for _ in range(n):
            self.queue.append((None, None))

    def wait(self, n):
        while len(self.queue) > n:
            buf, content = self.queue.pop(0)
            if buf is not None and all(b != buf for b, _ in self.queue):
                self.completed.append((buf, content))

    def barrier(self):
        for buf, content in self.completed:
            self.visible[buf] = content
            if self.pending.get(buf) == content:
                del self.pending[buf]
        self.completed = []
        self.seg += 1

    def read(self, buf, content, kind):
        if self.visible.get(buf) != content:
            raise Violation(f"{kind}: buffer {buf} holds {self.visible.get(buf)}, "
                            f"expected {content}")
        if buf in self.pending:
            raise Violation(f"{kind}: buffer {buf} read with a load into it in flight")
        self.last_read[buf] = self.seg
        self.reads.append((kind, content))

    # the wave's own staging area: visible as soon as this wave's loads completed
    def read_private(self, buf, content, kind):
        if any(b == buf for b, _ in self.queue):
            raise Violation(f"{kind}: staging area read with its loads in flight")
        done = [c for b, c in self.completed if b == buf]
        vis = done[-1] if done else self.visible.get(buf)
        if vis != content:
            raise Violation(f"{kind}: staging holds {vis}, expected {content}")
        self.completed = [(b, c) for b, c in self.completed if b != buf]
        self.visible[buf] = content
        self.pending.pop(buf, None)
        self.last_read[buf] = self.seg
        self.reads.append((kind, content))

    # the wave's own staging area as scratch: no load into it may be in flight
    def use_private(self, buf, kind):
        if any(b == buf for b, _ in self.queue):
            raise Violation(f"{kind}: staging area reused with a load into it in flight")
        if self.pending.get(buf) is not None and any(b == buf for b, _ in self.completed):
            raise Violation(f"{kind}: staging area reused before its loaded rows were read")
        self.last_read[buf] = self.seg

    def write_table(self, slot, unit):
        buf = ("tab", slot)
        if unit >= self.J:
            raise Violation("table of a unit past the last one")
        if self.last_read.get(buf, -1) >= self.seg:
            raise Violation(f"table {slot} rewritten in the segment where it is read")
        self.pending[buf] = ("tab", unit)
        self.completed.append((buf, ("tab", unit)))   # plain LDS stores: done at once

    def read_table(self, slot, unit, kind):
        self.read(("tab", slot), ("tab", unit), kind)


def run_schedule(nkt, J, KD, ipw=2, QI=8):
    """Walks the kernel's schedule for one workgroup of J units of nkt key
    tiles (nkt even, at least 4) with KD K buffers."""
    assert nkt >= 4 and nkt % 2 == 0
    M = Model(nkt, J, KD, ipw, QI)
    qstep = nkt - 2
    kb0 = 0

    def kslot(pos):
        return pos % 2 if KD == 2 else (kb0 + pos) % KD

    def K(b):
        return ("K", b)

    def V(b):
        return ("V", b)

    def dma(kind, buf, unit, tile):
        # a window tile's rows are addressed through its unit's table
        M.read_table(unit % 2, unit, f"{kind} tile offsets")
        M.issue(buf, (kind, unit, tile), ipw)

    # ---- unit 0: tables of units 0 and 1, then its first tiles
    M.write_table(0, 0)
    if J > 1:
        M.write_table(1, 1)
    M.barrier()
    M.read_table(0, 0, "Q rows of unit 0")          # Q of unit 0 straight to registers
    M.queue.append((None, None))
    dma("K", K(0), 0, 0)
    dma("V", V(0), 0, 0)
    dma("K", K(1), 0, 1)
    if KD == 3:
        dma("K", K(2), 0, 2)
    M.wait(0)
    M.barrier()
    M.read(K(kslot(0)), ("K", 0, 0), "S(0)")

    for j in range(J):
        has_next = j + 1 < J
        uc, un = j, j + 1
        M.barrier()                                   # unit top
        dma("V", V(1), uc, 1)
        dma("K", K(kslot(KD)), uc, KD)
        if j >= 1 and has_next:
            M.write_table((j + 1) % 2, j + 1)

        for t in range(nkt - 1):
            M.read(K(kslot(t + 1)), ("K", uc, t + 1), f"S({t + 1})")
            M.read(V(t % 2), ("V", uc, t), f"PV({t})")
            if KD == 3:
                M.wait(ipw if (t + 3 < nkt or has_next) else 0)
            else:
                M.wait(0)
            M.barrier()
            tv, tk = t + 2, t + 1 + KD
            do_v = tv < nkt or (has_next and tv == nkt)
            do_k = tk < nkt or (has_next and tk < nkt + KD)
            if KD == 3 and has_next and t < qstep:
                for i in range(t, QI, qstep):
                    M.read_table(un % 2, un, "Q staging rows")
                    M.issue(("Q", i), ("Q", un, i))
            if do_v:
                dma("V", V(tv % 2), uc if tv < nkt else un, tv if tv < nkt else 0)
            if do_k:
                dma("K", K(kslot(tk)), uc if tk < nkt else un, tk if tk < nkt else tk - nkt)
            if KD == 2 and has_next and t < qstep:
                for i in range(t, QI, qstep):
                    M.read_table(un % 2, un, "Q staging rows")
                    M.issue(("Q", i), ("Q", un, i))
        t = nkt - 1
        M.read(V(t % 2), ("V", uc, t), f"PV({t})")
        if not has_next:
            M.read_table(uc % 2, uc, "output rows")
            for i in range(QI):
                M.use_private(("Q", i), "output staging")
            M.store(8)
            break
        M.wait(ipw if KD == 3 else 0)
        for i in range(QI):
            M.read_private(("Q", i), ("Q", un, i), "Q of the next unit")
        M.read(K(kslot(nkt)), ("K", un, 0), "S(0) of the next unit")
        M.read_table(uc % 2, uc, "output rows")
        for i in range(QI):
            M.use_private(("Q", i), "output staging")
        M.store(8)
        if KD == 3:
            kb0 = (kb0 + nkt) % KD
    M.wait(0)
    if M.queue:
        raise Violation("operations left in flight at the end")
    return M


WALKS = [(nkt, J) for nkt in (4, 6, 8, 10, 16, 20, 24, 40, 80) for J in (1, 2, 3, 4, 7)]


@pytest.mark.parametrize("KD", [2, 3])
@pytest.mark.parametrize("nkt,J", WALKS)
def test_schedule_is_race_free(nkt, J, KD):
    for ipw, QI in ((2, 8), (1, 4)):                  # head dim 128 and 64
        M = run_schedule(nkt, J, KD, ipw, QI)
        # every unit reads each of its key tiles once as K and once as V, in order
        for kind in ("K", "V"):
            seen = [c for k, c in M.reads if c[0] == kind]
            assert seen == [(kind, j, t) for j in range(J) for t in range(nkt)]


@pytest.mark.parametrize("KD", [2, 3])
def test_model_catches_a_late_wait(KD, monkeypatch):
    # waiting for one operation fewer than the schedule needs must be caught
    orig = Model.wait

    def short_wait(self, n):
        orig(self, n + 1)

    monkeypatch.setattr(Model, "wait", short_wait)
    with pytest.raises(Violation):
        run_schedule(8, 3, KD)


def test_model_catches_a_load_into_a_buffer_being_read():
    M = Model(8, 1, 2, 2, 8)
    M.issue(("K", 0), ("K", 0, 0), 2)
    M.wait(0)
    M.barrier()
    M.read(("K", 0), ("K", 0, 0), "S(0)")
    with pytest.raises(Violation):
        M.issue(("K", 0), ("K", 0, 2), 2)             # same segment as the read


def test_model_catches_output_staging_over_a_staging_load():
    # the output rows may not go through the staging area while the next
    # unit's Q rows are still being loaded into it
    M = Model(8, 2, 2, 2, 8)
    M.issue(("Q", 0), ("Q", 1, 0))
    with pytest.raises(Violation, match="output staging"):
        M.use_private(("Q", 0), "output staging")


def test_model_catches_a_load_past_the_last_unit():
    M = Model(8, 2, 3, 2, 8)
    with pytest.raises(Violation):
        M.issue(("K", 1), ("K", 2, 0), 2)
