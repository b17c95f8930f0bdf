"""Model of the kernels' Top-K threshold search (topk.hip, decode.hip), on the
CPU: keys sit 16 to a lane over 64 lanes (0 for non-candidates), the threshold
is the largest t with #(keys >= t) >= K.  The kernels first take t0 = the K-th
largest lane maximum, then search only the keys >= t0 when they fit one per
lane.  This checks that the two-stage search gives the plain search's
threshold on random, tie-heavy and small-range inputs."""
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
