"""Model of the kernels' Top-K threshold search (topk.hip, decode.hip), on the
CPU: keys sit 16 to a lane over 64 lanes (0 for non-candidates), the threshold
is the largest t with #(keys >= t) >= K.  The kernels first take t0 = the K-th
largest lane maximum, then search only the keys >= t0 when they fit one per
lane.  This checks that the two-stage search gives the plain search's
threshold on random, tie-heavy and small-range inputs, and that the prefill
kernel's whole selection (its 16-bit bound, the count of keys at or above
the threshold over the gathered keys, the take-all path when exactly K keys
reach the threshold and the tie path otherwise) selects the K largest keys
with ties to the lower index."""
import numpy as np
import pytest


def plain_threshold(keys, K):
    thr = 0
    for bit in range(31, -1, -1):
        cand = thr | (1 << bit)
        if int((keys >= cand).sum()) >= K:
            thr = cand
    return thr


def two_stage_threshold(keys2d, K):
    """keys2d [E, 64]: register e of lane l holds candidate l + 64 e."""
    lmax = keys2d.max(axis=0)
    t0 = plain_threshold(lmax, K)            # one value per lane
    above = keys2d[keys2d >= t0]
    if above.size > 64:
        return plain_threshold(keys2d.ravel(), K), True
    return plain_threshold(above, K), False


@pytest.mark.parametrize("kind", ["random32", "ties", "normal", "small_c"])
def test_two_stage_threshold_matches_plain(kind):
    rng = np.random.default_rng({"random32": 1, "ties": 2, "normal": 3, "small_c": 4}[kind])
    fallbacks = 0
    for _ in range(600):
        K = int(rng.integers(1, 64))
        hi = 65 if kind == "small_c" else 1025
        c = int(rng.integers(K + 1, max(K + 2, hi)))     # c > K historical candidates
        if kind == "ties":
            vals = rng.integers(1, 40, size=c)
        elif kind == "random32":
            vals = rng.integers(1, 2 ** 32 - 1, size=c, dtype=np.int64)
        else:
            vals = (np.abs(rng.standard_normal(c)) * 1e4).astype(np.int64) + 1
        keys = np.zeros(16 * 64, dtype=np.int64)
        keys[:c] = vals
        thr, fb = two_stage_threshold(keys.reshape(16, 64), K)
        fallbacks += fb
        assert thr == plain_threshold(keys, K)
    if kind in ("random32", "normal"):
        assert fallbacks < 600                       # the bound usually applies


def kernel_selection(keys2d, c, K):
    """The prefill kernel's whole selection as it runs per row: the bound t0k
    (the K-th largest lane maximum with its low 16 bits cleared, found by a
    search over the top 16 bits), the gathered keys >= t0k when they fit one
    per lane, the threshold, the count of keys >= threshold (over the
    gathered keys alone on that path), then either every key >= threshold
    (exactly K of them) or the keys above it plus the lowest-index equal
    keys.  Returns the selected candidate indices in ascending order."""
    E = keys2d.shape[0]
    flat = keys2d.ravel()                       # index l + 64 e -> keys2d[e, l]
    lmax = keys2d.max(axis=0)
    t0k = 0
    for bit in range(31, 15, -1):
        cand = t0k | (1 << bit)
        if int((lmax >= cand).sum()) >= K:
            t0k = cand
    gathered = flat[flat >= t0k]
    if gathered.size <= 64:
        thr = plain_threshold(gathered, K)
        n_ge = int((gathered >= thr).sum())
    else:
        thr = plain_threshold(flat, K)
        n_ge = int((flat >= thr).sum())
    idx = np.arange(E * 64)
    hist = idx < c
    if n_ge == K:
        sel = hist & (flat >= thr)
    else:
        gt = hist & (flat > thr)
        eq = np.flatnonzero(hist & (flat == thr))
        sel = gt.copy()
        sel[eq[:K - int(gt.sum())]] = True
    return np.flatnonzero(sel)


def reference_selection(vals, K):
    """The K largest keys, equal keys to the lower index, ascending."""
    order = sorted(range(len(vals)), key=lambda j: (-int(vals[j]), j))
    return np.array(sorted(order[:K]))


@pytest.mark.parametrize("kind", ["random32", "ties", "normal", "small_c"])
def test_kernel_selection_matches_reference(kind):
    """The fast path (exactly K keys at or above the threshold) and the tie
    path together select the K largest keys with ties to the lower index."""
    rng = np.random.default_rng({"random32": 11, "ties": 12, "normal": 13, "small_c": 14}[kind])
    fast = 0
    for _ in range(400):
        K = int(rng.integers(1, 64))
        hi = 65 if kind == "small_c" else 1025
        c = int(rng.integers(K + 1, max(K + 2, hi)))
        if kind == "ties":
            vals = rng.integers(1, 40, size=c)
        elif kind == "random32":
            vals = rng.integers(1, 2 ** 32 - 1, size=c, dtype=np.int64)
        else:
            vals = (np.abs(rng.standard_normal(c)) * 1e4).astype(np.int64) + 1
        E = -(-(c + 1) // 64)
        keys = np.zeros(E * 64, dtype=np.int64)
        keys[:c] = vals
        got = kernel_selection(keys.reshape(E, 64), c, K)
        want = reference_selection(vals, K)
        assert got.tolist() == want.tolist()
        thr = plain_threshold(keys, K)
        fast += int((keys >= thr).sum()) == K
    if kind == "ties":
        assert fast < 400                            # the tie path runs
    else:
        assert fast > 0                              # the fast path runs
