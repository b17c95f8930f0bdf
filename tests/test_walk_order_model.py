"""CPU model of the staging order of the query-group walks (walk_order.hip,
used by the forward and dQ kernels), and GPU checks of the kernel against it.

A walk takes a group of tpw consecutive tokens of one selection head
(tpw = min(64, 14 TPT), tiles of TPT tokens) and copies the union of their
selected blocks through a small LDS ring; the order decides how evenly each
tile's blocks fall into the ring's windows.  The model:
  * union blocks ascending, mask[p] = the tiles whose tokens selected block p;
  * candidates: the first 64 unplaced union positions, ranked by (largest
    window load among its tiles, 64 - tiles needing it, position), the window
    being the last three placed blocks; each step ranks them once and places
    up to two: the best, then the best whose tiles are disjoint from the
    first's.
CPU tests check the model (a permutation of the union, better-balanced
windows than ascending order on random selections, edge cases); GPU tests
compare the kernel's order with the model bit-exactly (integer work).
"""
import numpy as np
import pytest
import torch

import synth

WIN = 4
PICK = 2


def walk_tpw(TPT):
    return min(64, 14 * TPT)


def union_and_masks(sel_rows, t0, TPT):
    """sel_rows [ntok, S] block indices of the group's tokens -> ascending
    union blocks and per-block tile masks (entries outside 0..c(t) ignored)."""
    need = {}
    for tl, row in enumerate(sel_rows):
        c = (t0 + tl) // 64
        for j in row:
            j = int(j)
            if 0 <= j <= c:
                need[j] = need.get(j, 0) | (1 << (tl // TPT))
    blocks = sorted(need)
    return blocks, [need[j] for j in blocks]


def place(masks):
    """Placement order (union positions) for the tile masks of the union."""
    nU = len(masks)
    left = list(range(nU))
    cnt = {}
    hist = []
    out = []

    def push(p):
        if len(hist) == WIN - 1:
            old = hist.pop(0)
            for w in range(16):
                if masks[old] >> w & 1:
                    cnt[w] -= 1
        hist.append(p)
        for w in range(16):
            if masks[p] >> w & 1:
                cnt[w] = cnt.get(w, 0) + 1
        out.append(p)
        left.remove(p)

    while left:
        cand = left[:64]

        def key(p):
            m = masks[p]
            ml = max(cnt.get(w, 0) for w in range(16) if m >> w & 1)
            return (ml, 64 - bin(m).count("1"), p)
        picks, used = [], 0
        for q in sorted(cand, key=key):
            if masks[q] & used == 0:
                picks.append(q)
                used |= masks[q]
                if len(picks) == PICK:
                    break
        for q in picks:
            push(q)
    return out


def model_orders(idx, TPT):
    """idx [B,T,Hs,S] (numpy) -> {group index: list of blocks in order}."""
    B, T, Hs, S = idx.shape
    tpw = walk_tpw(TPT)
    ngrp = -(-T // tpw)
    res = {}
    for b in range(B):
        for sg in range(Hs):
            for grp in range(ngrp):
                t0 = grp * tpw
                rows = idx[b, t0:min(T, t0 + tpw), sg]
                blocks, masks = union_and_masks(rows, t0, TPT)
                res[(b * Hs + sg) * ngrp + grp] = [blocks[p] for p in place(masks)]
    return res


def window_max_loads(masks, order):
    """Mean over windows of WIN consecutive placed blocks of the busiest
    tile's count of needed blocks."""
    loads = []
    for i in range(len(order) - WIN + 1):
        cnt = {}
        for p in order[i:i + WIN]:
            for w in range(16):
                if masks[p] >> w & 1:
                    cnt[w] = cnt.get(w, 0) + 1
        loads.append(max(cnt.values()))
    return float(np.mean(loads))


def random_group(rng, c, K=31, ntok=56, t0=None):
    t0 = c * 64 if t0 is None else t0
    rows = []
    for tl in range(ntok):
        cc = (t0 + tl) // 64
        h = rng.choice(cc, min(K, cc), replace=False) if cc > 0 else np.zeros(0, int)
        rows.append(np.concatenate([np.sort(h), [cc], -np.ones(K - len(h), int)]))
    return np.array(rows), t0


# ------------------------------------------------------------------ CPU model


@pytest.mark.parametrize("c", [0, 3, 40, 300, 511])
def test_order_is_a_permutation_of_the_union(c):
    rng = np.random.default_rng(c)
    rows, t0 = random_group(rng, c)
    blocks, masks = union_and_masks(rows, t0, 4)
    order = place(masks)
    assert sorted(order) == list(range(len(blocks)))
    assert len(blocks) == len(set(int(j) for r in rows for j in r if 0 <= j <= (t0 + 55) // 64))


def test_order_balances_the_ring_windows():
    """On random selections late in a 32K sequence the busiest tile of a
    ring window needs fewer of its blocks than in ascending order."""
    rng = np.random.default_rng(11)
    asc, placed = [], []
    for c in (256, 400, 511):
        rows, t0 = random_group(rng, c)
        _, masks = union_and_masks(rows, t0, 4)
        asc.append(window_max_loads(masks, list(range(len(masks)))))
        placed.append(window_max_loads(masks, place(masks)))
    assert all(p < 0.85 * a for p, a in zip(placed, asc)), (asc, placed)


def test_small_unions_and_empty_rows():
    # every token only selects its current block: union = the group's blocks
    rows = np.full((56, 4), -1)
    rows[:, 0] = [(40 + t) // 64 for t in range(56)]
    blocks, masks = union_and_masks(rows, 40, 4)
    assert blocks == [0, 1] and masks == [0x3F, 0x3FC0]
    assert sorted(place(masks)) == [0, 1]
    # no valid entry at all
    assert union_and_masks(np.full((56, 4), -1), 0, 4) == ([], [])
    assert place([]) == []
    # a future block (beyond the token's current block) is ignored
    rows = np.array([[0, 5]] + [[0, -1]] * 13)
    assert union_and_masks(rows, 0, 4)[0] == [0]


def test_window_rule_matches_the_plain_definition():
    """Each step's placements are, in turn, the best candidate by a recount
    of the window (the last three blocks placed before the step) among those
    whose tiles are disjoint from the step's earlier picks, at most PICK per
    step (a check of the model's bookkeeping)."""
    rng = np.random.default_rng(5)
    rows, t0 = random_group(rng, 200)
    _, masks = union_and_masks(rows, t0, 4)
    order = place(masks)
    left = list(range(len(masks)))

    def key(q, window):
        ml = max(sum(1 for r in window if masks[r] >> w & 1)
                 for w in range(16) if masks[q] >> w & 1)
        return (ml, 64 - bin(masks[q]).count("1"), q)
    n = 0
    while n < len(order):
        window = order[max(0, n - (WIN - 1)):n]
        cand = left[:64]
        used = 0
        for _ in range(PICK):
            rest = [q for q in cand if masks[q] & used == 0]
            if not rest:
                break
            p = min(rest, key=lambda q: key(q, window))
            assert order[n] == p
            used |= masks[p]
            left.remove(p)
            n += 1


# ------------------------------------------------------------------ GPU kernel

CASES = [
    # (T, Hq, Hkv, K, per-query-head)
    (1000, 8, 2, 3, False),
    (4096, 40, 8, 15, False),
    (8192, 32, 8, 31, False),
    (1000, 4, 2, 7, True),
    (2500, 16, 2, 31, False),   # G = 8: TPT = 2
]


@pytest.mark.gpu
@pytest.mark.parametrize("T,Hq,Hkv,K,pq", CASES)
def test_kernel_order_matches_model(T, Hq, Hkv, K, pq):
    import gated_block_sparse_gate_amd as sas
    w = synth.Workload(f"walk_T{T}", 77, B=1, T=T, Hq=Hq, Hkv=Hkv, D=128, dg=128, topk=K,
                       kind="train", gate="q" if pq else "kv")
    idx, _ = synth.random_selection(w, seed=3, K=K)
    idx = idx.contiguous()
    Gs = 1 if pq else Hq // Hkv
    TPT = 16 // Gs
    print(f"walk order T={T} Hq={Hq} Hkv={Hkv} K={K} per-query-head={pq}", flush=True)
    got = sas.walk_order(idx.cuda(), Hq, Hkv).cpu().numpy().view(np.uint16)
    ref = model_orders(idx.numpy(), TPT)
    assert got.shape[0] == len(ref)
    for g, blocks in ref.items():
        n = int(got[g, 0])
        assert n == len(blocks), (g, n, len(blocks))
        assert got[g, 1:1 + n].tolist() == blocks, g
