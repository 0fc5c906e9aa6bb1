"""The safe pruning of the ROCmFP4 scale search (ROCmFP4 design page, section 03: pruning may skip only work
that cannot change the selected scale), checked on the CPU against the oracle's exhaustive search.

The device packer visits the finite UE4M3 codes outward from the start code and drops a direction once a
lower bound of the error reaches the best error found. The bounds are sums of some of E(c)'s own terms:
  down (smaller scales): weights with |w| > 10 s, which take level 10: v (|w| - 10 s)^2;
  up (larger scales):    weights with |w| <= s / 2, which take level 0:  v w^2.
Pinned here, for random and adversarial groups of 16 and 32 weights, with and without importance:
  * each bound is <= the oracle's E(c) for every code (summed in the same index order);
  * the down bound never shrinks as the code falls and the up bound never shrinks as it rises;
  * the pruned visit order selects exactly the exhaustive winner under (E, |c - start|, c).
"""
import numpy as np
import pytest

import synth
from oracle import formats, pack

CODES = np.arange(formats.UE4M3_FINITE_CODES)
SCALES = formats.ue4m3_value(CODES.astype(np.uint8))


def _seq_sum(terms):
    """Sum in index order along the last axis (np.cumsum is sequential; its last element is the sum)."""
    return np.cumsum(terms, axis=-1)[..., -1]


def bounds(w, v):
    """(down, up) bounds for every code: arrays [groups, 127]."""
    a = np.abs(w.astype(np.float64))[:, None, :]                 # [G, 1, g]
    s = SCALES[None, :, None]                                    # [1, 127, 1]
    vv = np.ones_like(a) if v is None else v.astype(np.float64)[:, None, :]
    dlt = a - 10.0 * s
    down = np.where(a > 10.0 * s, vv * (dlt * dlt), 0.0)
    up = np.where(a <= 0.5 * s, vv * (a * a), 0.0)
    return _seq_sum(down), _seq_sum(up)


def start_code(w):
    amax = np.max(np.abs(w.astype(np.float64)), axis=1)
    return formats.e4m3_encode_rne(np.minimum(amax / 10.0, 448.0)).astype(np.int64)


def pruned_search(e_row, bd, bu, start):
    """The device packer's visit order with pruning, on one group's error table."""
    best_c, best_e = start, e_row[start]
    down = up = True
    scored = 1
    for d in range(1, 127):
        if not (down or up):
            break
        for c, alive_is_down in ((start - d, True), (start + d, False)):
            if alive_is_down and not down or (not alive_is_down) and not up:
                continue
            if c < 0 or c > 126:
                if alive_is_down:
                    down = False
                else:
                    up = False
                continue
            b = bd[c] if alive_is_down else bu[c]
            if b >= best_e:
                if alive_is_down:
                    down = False
                else:
                    up = False
                continue
            scored += 1
            e = e_row[c]
            key, bkey = (e, abs(c - start), c), (best_e, abs(best_c - start), best_c)
            if key < bkey:
                best_c, best_e = c, e
    return best_c, scored


def groups(kind, g, count, seed):
    rng = np.random.default_rng(seed)
    if kind == "t":
        w = synth.weights(count, g, dist="t", nu=4.0, cfg=120, mat=seed)
    elif kind == "outlier":
        w = synth.weights(count, g, dist="t", nu=4.0, outlier_frac=0.05, cfg=121, mat=seed)
    elif kind == "levels":   # weights on or near grid points and midpoints of a random scale
        s = formats.ue4m3_value(rng.integers(1, 127, size=(count, 1)).astype(np.uint8))
        mult = rng.choice([0, 0.5, 1, 1.5, 2, 2.5, 3, 3.5, 4, 5, 6, 7, 8, 9, 10, 11, 40], size=(count, g))
        w = (mult * s * rng.choice([-1, 1], size=(count, g))).astype(np.float32)
    else:                    # tiny, huge and zero groups
        w = np.zeros((count, g), np.float32)
        w[0::3] = 1e-7 * rng.standard_normal((len(w[0::3]), g))
        w[1::3] = 4000.0 * rng.standard_normal((len(w[1::3]), g))
    return w.astype(np.float32)


@pytest.mark.parametrize("g", [16, 32])
@pytest.mark.parametrize("kind", ["t", "outlier", "levels", "extreme"])
@pytest.mark.parametrize("weighted", [False, True])
def test_bounds_and_pruned_winner(g, kind, weighted):
    count = 400
    w = groups(kind, g, count, seed=g + 7)
    v = None
    if weighted:
        rng = np.random.default_rng(3)
        v = np.abs(rng.standard_normal((count, g))).astype(np.float32)
        v[rng.random((count, g)) < 0.2] = 0.0                        # some weights unimportant
    e = pack.rocmfp4_all_errors(w, v)                                 # the oracle's E(c), [count, 127]
    bd, bu = bounds(w, v)
    assert np.all(bd <= e) and np.all(bu <= e)
    assert np.all(np.diff(bd, axis=1) <= 0)                           # grows as the code falls
    assert np.all(np.diff(bu, axis=1) >= 0)                           # grows as the code rises
    _, want, _ = pack.rocmfp4_search(w, v)
    starts = start_code(w)
    scored = []
    for i in range(count):
        c, n = pruned_search(e[i], bd[i], bu[i], int(starts[i]))
        assert c == want[i], (i, c, want[i])
        scored.append(n)
    # pruning has to skip work to be worth it: far fewer than 127 candidates scored on these groups
    assert np.mean(scored) < 60
