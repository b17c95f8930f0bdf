"""CPU event model of the staging protocol with dedicated stager waves
(dQ kernel, attn_bwd.hip), checked on random interleavings.

Stager waves copy blocks in order into ring slot n % R with asynchronous
copies (up to L < R blocks in flight each, so two blocks of one slot are
never in flight together; copies may land in any order).  Before copying block n a stager waits
until every compute wave's progress word is >= n - R + 1 (all are done with
the slot's previous block); it bumps fill[n % R] once its copies of block n
have landed, and publishes everything in flight before it waits.  A compute
wave visits only the blocks its tile needs: it waits until
fill[v % R] >= S * (v // R + 1), reads the slot, then sets its progress word to
its next needed block (or nU).  Checks: no deadlock, no read before all parts
landed, no part landing in a slot a compute wave still reads.

The forward (attn_fwd.hip) splits the slot into one ring per stager (K, V^T):
stager s fills ring s and waits on the compute waves' progress words of ring s
only; a compute wave reads a block's part in ring 0, sets its ring-0 progress
word to its next needed block, then reads the part in ring 1, and so on
(run_split).
"""
import random

import pytest


def run(S, C, R, L, nU, seed, p_act=0.3, free_slack=0, ready_slack=0):
    rnd = random.Random(seed)
    act = [[rnd.random() < p_act for _ in range(nU)] for _ in range(C)]
    fill = [0] * R
    held = [[None] * S for _ in range(R)]
    readers = [set() for _ in range(R)]

    def next_act(c, v):
        while v < nU and not act[c][v]:
            v += 1
        return v

    prog = [next_act(c, 0) for c in range(C)]
    comp = [dict(v=prog[c], st="wait", busy=0) for c in range(C)]
    stag = [dict(n=0, inflight=[], st="run") for _ in range(S)]
    t = 0
    while any(x["v"] < nU for x in comp) or any(s["n"] < nU or s["inflight"] for s in stag):
        t += 1
        assert t < 2_000_000, ("deadlock", prog, fill, [(s["n"], len(s["inflight"])) for s in stag])
        order = [("c", i) for i in range(C)] + [("s", i) for i in range(S)]
        rnd.shuffle(order)
        for kind, i in order:
            if kind == "s":
                x = stag[i]
                for blk, tl in list(x["inflight"]):         # copies land
                    if tl <= t:
                        sl = blk % R
                        assert not readers[sl], ("part landed in a slot being read", blk)
                        held[sl][i] = blk
                        x["inflight"].remove((blk, tl))
                        x.setdefault("landed", []).append(blk)
                # publish landed blocks in order (s_waitcnt semantics: oldest first)
                landed = sorted(x.get("landed", []))
                while landed and (not x["inflight"] or landed[0] < min(b for b, _ in x["inflight"])):
                    fill[landed.pop(0) % R] += 1
                x["landed"] = landed
                n = x["n"]
                if n >= nU:
                    continue
                if min(prog) >= n - R + 1 - free_slack and len(x["inflight"]) < L:
                    x["inflight"].append((n, t + rnd.randint(2, 50)))
                    x["n"] += 1
            else:
                x = comp[i]
                if x["v"] >= nU:
                    continue
                if x["busy"] > 0:
                    x["busy"] -= 1
                    if x["busy"] == 0:
                        sl = x["v"] % R
                        assert all(b == x["v"] for b in held[sl]), ("slot changed while read", x["v"])
                        readers[sl].discard(i)
                        x["v"] = next_act(i, x["v"] + 1)
                        prog[i] = x["v"]
                    continue
                v, sl = x["v"], x["v"] % R
                if fill[sl] >= S * (v // R + 1) - ready_slack:
                    assert all(b == v for b in held[sl]), ("read before all parts landed", v, held[sl])
                    readers[sl].add(i)
                    x["busy"] = rnd.randint(1, 30)


def run_split(S, C, R, L, nU, seed, p_act=0.3, free_slack=0, ready_slack=0):
    rnd = random.Random(seed)
    act = [[rnd.random() < p_act for _ in range(nU)] for _ in range(C)]
    fill = [[0] * R for _ in range(S)]
    held = [[None] * R for _ in range(S)]
    readers = [[set() for _ in range(R)] for _ in range(S)]

    def next_act(c, v):
        while v < nU and not act[c][v]:
            v += 1
        return v

    prog = [[next_act(c, 0) for c in range(C)] for _ in range(S)]
    comp = [dict(v=prog[0][c], part=0, busy=0) for c in range(C)]
    stag = [dict(n=0, inflight=[], landed=[]) for _ in range(S)]
    t = 0
    while any(x["v"] < nU for x in comp) or any(s["n"] < nU or s["inflight"] for s in stag):
        t += 1
        assert t < 2_000_000, ("deadlock", prog, fill)
        order = [("c", i) for i in range(C)] + [("s", i) for i in range(S)]
        rnd.shuffle(order)
        for kind, i in order:
            if kind == "s":
                x = stag[i]
                for blk, tl in list(x["inflight"]):
                    if tl <= t:
                        sl = blk % R
                        assert not readers[i][sl], ("part landed in a slot being read", i, blk)
                        held[i][sl] = blk
                        x["inflight"].remove((blk, tl))
                        x["landed"].append(blk)
                landed = sorted(x["landed"])
                while landed and (not x["inflight"] or landed[0] < min(b for b, _ in x["inflight"])):
                    fill[i][landed.pop(0) % R] += 1
                x["landed"] = landed
                n = x["n"]
                if n < nU and min(prog[i]) >= n - R + 1 - free_slack and len(x["inflight"]) < L:
                    x["inflight"].append((n, t + rnd.randint(2, 50)))
                    x["n"] += 1
            else:
                x = comp[i]
                if x["v"] >= nU:
                    continue
                v, p, sl = x["v"], x["part"], x["v"] % R
                if x["busy"] > 0:
                    x["busy"] -= 1
                    if x["busy"] == 0:
                        assert held[p][sl] == v, ("slot changed while read", p, v)
                        readers[p][sl].discard(i)
                        prog[p][i] = next_act(i, v + 1)      # released this ring's slot
                        if p + 1 < S:
                            x["part"] = p + 1
                        else:
                            x["part"] = 0
                            x["v"] = prog[p][i]
                    continue
                if fill[p][sl] >= v // R + 1 - ready_slack:
                    assert held[p][sl] == v, ("read before the part landed", p, v, held[p][sl])
                    readers[p][sl].add(i)
                    x["busy"] = rnd.randint(1, 30)


@pytest.mark.parametrize("S,C", [(2, 14), (2, 8), (3, 12)])
@pytest.mark.parametrize("R", [2, 4])
def test_split_rings_random_interleavings(S, C, R):
    for L in (1, 3):
        if L >= R:
            continue
        for nU in (0, 1, 2, 5, 17, 40):
            for seed in range(4):
                run_split(S, C, R, L, nU, seed)


@pytest.mark.parametrize("free_slack,ready_slack", [(1, 0), (0, 1)])
def test_split_rings_off_by_one_fails(free_slack, ready_slack):
    caught = False
    for seed in range(40):
        try:
            run_split(2, 14, 4, 1, 40, seed, p_act=0.6, free_slack=free_slack,
                      ready_slack=ready_slack)
        except AssertionError:
            caught = True
            break
    assert caught


@pytest.mark.parametrize("S,C", [(1, 8), (2, 14), (4, 12)])
@pytest.mark.parametrize("R", [2, 4, 8])
def test_stager_protocol_random_interleavings(S, C, R):
    for L in (1, 3):
        if L >= R:
            continue
        for nU in (0, 1, 2, 5, 17, 40):
            for seed in range(4):
                run(S, C, R, L, nU, seed)


@pytest.mark.parametrize("free_slack,ready_slack", [(1, 0), (0, 1)])
def test_stager_protocol_off_by_one_fails(free_slack, ready_slack):
    """Loosening either condition by one must be caught by the model."""
    caught = False
    for seed in range(40):
        try:
            run(2, 14, 4, 3, 40, seed, p_act=0.6, free_slack=free_slack,
                ready_slack=ready_slack)
        except AssertionError:
            caught = True
            break
    assert caught
