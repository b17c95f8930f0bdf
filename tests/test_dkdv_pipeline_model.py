"""CPU model of the dK/dV kernel's LDS schedule (attn_bwd.hip, dkdv_kernel).

The kernel streams tile pairs it = 0 .. nit-1 through LDS with one workgroup
barrier at the end of every pair.  Inside a pair the four waves run in any
order relative to each other, so between two barriers a location may be read
or written by several waves but never both written and read (or written
twice).  Per pair `it` the kernel accesses:

* reads: the Q / dO row tiles of pair it (buffer it % 2), the row metadata of
  pair it (slot it % NM), the metadata source rows of pair it + 1 (for the
  row prefetch), and the dS tile, dS row sums and entries of pair it - 1 (the
  dS stores of the previous pair);
* writes: the dS tile and row sums of pair it (tile it % ND), the metadata of
  pair it + 2 (slot (it + 2) % NM), and the Q / dO rows of pair it + 1
  (buffer (it + 1) % 2).

With MID set a barrier also separates the first part of the pair (S, dP and
the stores of pair it - 1) from the second (dS into LDS, metadata and row
stores), the form with NM = 3 metadata slots and ND = 1 dS tile.  The model
checks that no phase holds a race and that every read returns the data of the
pair it is meant for.
"""
import pytest


def run(nit, NM, ND, MID):
    # location -> (pair tag of the data it holds, phase of the last write)
    mem = {}
    phase = 0
    acc = {}                # location -> list of (kind, pair) in this phase

    def barrier():
        nonlocal phase, acc
        for loc, ops in acc.items():
            kinds = {k for k, _ in ops}
            writes = [p for k, p in ops if k == "w"]
            assert not ("w" in kinds and "r" in kinds), ("read and write in one phase", loc, ops)
            assert len(writes) <= 1 or len(set(writes)) == 1, ("two writes in one phase", loc, ops)
        acc = {}
        phase += 1

    def write(loc, pair):
        acc.setdefault(loc, []).append(("w", pair))
        mem[loc] = pair

    def read(loc, pair):
        acc.setdefault(loc, []).append(("r", pair))
        assert mem.get(loc) == pair, ("stale or early read", loc, pair, mem.get(loc))

    # prologue: metadata of pairs 0 and 1, barrier, rows of pair 0, barrier
    for p in (0, 1):
        if p < nit:
            write(("meta", p % NM), p)
    barrier()
    if nit > 0:
        read(("meta", 0), 0)
        write(("rows", 0), 0)
    barrier()
    for it in range(nit):
        # first part
        if it + 1 < nit:
            read(("meta", (it + 1) % NM), it + 1)        # row prefetch addresses
        if it > 0:
            read(("dsT", (it - 1) % ND), it - 1)         # dS stores of pair it - 1
            read(("meta", (it - 1) % NM), it - 1)
        read(("rows", it % 2), it)
        read(("meta", it % NM), it)
        if MID:
            barrier()
        # second part
        write(("dsT", it % ND), it)
        read(("rows", it % 2), it)                       # dK, dV operands
        if it + 2 < nit:
            write(("meta", (it + 2) % NM), it + 2)
        if it + 1 < nit:
            write(("rows", (it + 1) % 2), it + 1)
        barrier()
    if nit > 0:
        read(("dsT", (nit - 1) % ND), nit - 1)
        read(("meta", (nit - 1) % NM), nit - 1)
    barrier()


@pytest.mark.parametrize("nit", [0, 1, 2, 3, 4, 5, 9, 40])
def test_schedule_without_mid_barrier(nit):
    run(nit, NM=4, ND=2, MID=False)


@pytest.mark.parametrize("nit", [0, 1, 2, 3, 4, 9])
def test_schedule_with_mid_barrier(nit):
    run(nit, NM=3, ND=1, MID=True)


@pytest.mark.parametrize("NM,ND", [(3, 2), (4, 1)])
def test_fewer_slots_without_mid_barrier_race(NM, ND):
    """Three metadata slots or one dS tile need the mid-pair barrier."""
    with pytest.raises(AssertionError):
        run(9, NM=NM, ND=ND, MID=False)
