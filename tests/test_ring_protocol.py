"""CPU event model of the LDS ring protocol of the query-block walks (forward
and dQ kernels, attn_fwd.hip / attn_bwd.hip), checked on random interleavings.

Per block u (slot u % R), each of NW waves:
  * writes its share of block n (held in registers, loaded from global memory
    with some latency) into slot n % R once done[n % R] >= NW * (n // R), then
    bumps fill[n % R] and starts loading its share of block n + 1; it tries
    this at every block boundary, in the middle of an active block, and on
    every poll while it waits;
  * waits until fill[u % R] >= NW * (u // R + 1), reads the slot (for a random
    time), bumps done[u % R].
Checks: every wave finishes (no deadlock), a block is read only when all NW
shares of it are in its slot, and no share lands in a slot while a wave still
reads the slot's previous block.  Host logic only: no GPU.
"""
import random

import pytest


def run(NW, R, nU, seed, act_p=0.3):
    rnd = random.Random(seed)
    fill = [0] * R
    done = [0] * R
    held = [[None] * NW for _ in range(R)]   # block whose share w sits in the slot
    readers = [set() for _ in range(R)]
    waves = [dict(u=0, nxt=0, ready=0, st="bnd", busy=0, mid=False) for _ in range(NW)]
    if nU == 0:
        return
    t = 0
    finished = 0

    def try_write(w):
        x = waves[w]
        n = x["nxt"]
        if n < nU and done[n % R] >= NW * (n // R) and x["ready"] <= t:
            s = n % R
            assert not readers[s], ("share written into a slot still being read", n)
            held[s][w] = n
            fill[s] += 1
            x["nxt"] += 1
            x["ready"] = t + rnd.randint(1, 40)     # load latency of the next share

    while finished < NW:
        t += 1
        assert t < 2_000_000, ("deadlock", [(x["u"], x["nxt"], x["st"]) for x in waves])
        for w in rnd.sample(range(NW), NW):
            x = waves[w]
            if x["st"] == "fin":
                continue
            if x["busy"] > 0:
                x["busy"] -= 1
                if x["mid"] and x["busy"] == 0:
                    x["mid"] = False
                    try_write(w)                   # the mid-block hand-over
                    x["busy"] = rnd.randint(5, 40)
                continue
            u, s = x["u"], x["u"] % R
            if x["st"] == "bnd":
                try_write(w)
                x["st"] = "wait"
            if x["st"] == "wait":
                if fill[s] >= NW * (u // R + 1):
                    assert all(b == u for b in held[s]), ("read before all shares landed", u)
                    readers[s].add(w)
                    x["st"] = "read"
                    if rnd.random() < act_p:
                        x["busy"], x["mid"] = rnd.randint(5, 40), True
                    else:
                        x["busy"] = rnd.randint(0, 2)
                else:
                    try_write(w)
                continue
            if x["st"] == "read":
                assert all(b == u for b in held[s]), ("slot overwritten while read", u)
                readers[s].discard(w)
                done[s] += 1
                x["u"] += 1
                x["st"] = "fin" if x["u"] == nU else "bnd"
                finished += x["st"] == "fin"


@pytest.mark.parametrize("NW", [8, 16])
@pytest.mark.parametrize("R", [2, 3, 4, 8])
def test_ring_protocol_random_interleavings(NW, R):
    for nU in (0, 1, 2, 3, 5, 9, 33):
        for seed in range(6):
            run(NW, R, nU, seed)
