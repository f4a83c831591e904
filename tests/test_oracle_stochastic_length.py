"""Pins for the Stochastic Length rule of the oracle (CPU only)."""

import math
import os

import numpy as np

from oracle import stochastic_length as sl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    out = {}
    with open(os.path.join(GOLDEN, "stochastic_length.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                out[k] = float(v)
    return out


def test_closed_forms_from_pages():
    g = _golden()
    N, a = int(g["N"]), g["alpha"]
    assert sl.subsample_length(N, a) == int(g["L"]) == 776
    for n in (4096, 2048, 1024):
        assert abs(sl.keep_probability(n, N, a) - g[f"p_keep_{n}"]) < 1e-9
    # always kept at or below the subsample length
    assert sl.keep_probability(776, N, a) == 1.0
    assert sl.keep_probability(777, N, a) < 1.0


def test_selection_shape_and_order():
    rng = np.random.default_rng(0)
    lengths = np.array([100, 776, 777, 4096, 3000, 0, 2000])
    off = np.concatenate([[0], np.cumsum(lengths)])
    u = rng.random(lengths.size)
    u[3] = 0.999  # force a cut
    u[4] = 0.0    # force a keep (p > 0)
    keys = rng.integers(0, 2**32, size=int(off[-1]), dtype=np.uint64).astype(np.uint32)
    kept, new_off = sl.select(off, u, keys)
    new_len = np.diff(new_off)
    for b, n in enumerate(lengths):
        seg = kept[new_off[b]:new_off[b + 1]]
        assert np.all(seg >= off[b]) and np.all(seg < off[b + 1])
        assert np.all(np.diff(seg) > 0)
        if n <= 776 or b == 4:
            assert new_len[b] == n
        elif b == 3:
            assert new_len[b] == 776
        else:
            assert new_len[b] in (n, 776)
    # the cut keeps exactly the 776 smallest priorities
    s0, s1 = off[3], off[4]
    seg = kept[new_off[3]:new_off[4]]
    thr = np.sort(keys[s0:s1])[775]
    assert np.all(keys[seg] <= thr)
    assert np.sum(keys[s0:s1] < thr) <= 775


def test_keep_rate_matches_binomial():
    rng = np.random.default_rng(1)
    for n in (1024, 2048, 4096):
        p = sl.keep_probability(n, 4096, 1.6)
        trials = 100_000
        u = rng.random(trials)
        # the rule only looks at u for the keep decision; use one token per user as a stub
        kept = sum(1 for x in u if x < sl.keep_threshold(n, 4096, 1.6))
        sigma = math.sqrt(trials * p * (1 - p))
        assert abs(kept - trials * p) < 5 * sigma


def test_subsample_is_uniform_over_positions():
    rng = np.random.default_rng(2)
    n, reps = 1600, 400
    counts = np.zeros(n)
    for _ in range(reps):
        keys = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
        kept, _ = sl.select(np.array([0, n]), np.array([0.999999]), keys)
        counts[kept] += 1
    # each position is kept with probability 776/1600
    p = 776 / n
    z = (counts - reps * p) / math.sqrt(reps * p * (1 - p))
    assert abs(z.mean()) < 0.2
    assert np.abs(z).max() < 5.5
