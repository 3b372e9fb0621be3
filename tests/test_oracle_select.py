"""Pins of the oracle's HKVD counts, schedule and top-k (CPU only)."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import blend


def test_num_selected_exact_ceiling():
    # 0.07 * 100 is 7.000000000000001 in binary floating point; exact is 7
    assert blend.num_selected(700, 100, 1000) == 7
    assert blend.num_selected(1500, 3072, 2560) == 461     # 460.8
    assert blend.num_selected(1500, 128, 64) == 20          # 19.2
    assert blend.num_selected(1500, 4000, 3500) == 600      # exact
    assert blend.num_selected(10000, 3072, 2560) == 2560    # capped by candidates
    assert blend.num_selected(0, 3072, 2560) == 0
    rng = np.random.default_rng(0)
    for _ in range(2000):
        r, n, c = int(rng.integers(0, 10001)), int(rng.integers(0, 20000)), int(rng.integers(0, 20000))
        want = min(-(-(r * n) // 10000), c)
        assert blend.num_selected(r, n, c) == want
        assert want == min(math.ceil(Fraction(r, 10000) * n), c)


def test_filter_schedule_stack_workload():
    ks = blend.filter_schedule(32, 3000, 1500, 4096, 3584)
    assert ks[0] == 3584 and ks[1] == 1229 and ks[-1] == 615
    assert all(a >= b for a, b in zip(ks[1:], ks[2:]))
    # linear in r: layer 16 sits at r = 0.30 - 0.15 * 15/30 = 0.225 -> ceil(921.6)
    assert ks[16] == 922


def test_filter_schedule_constant_ratio():
    ks = blend.filter_schedule(80, 1500, 0, 4000, 3500)
    assert ks[0] == 3500 and set(ks[1:]) == {600}


def _brute_topk(dev, k):
    best = None
    for sub in itertools.combinations(range(len(dev)), k):
        key = (sorted((dev[i] for i in sub), reverse=True), [-i for i in sub])
        # larger sorted-descending values first, then the smaller index set
        if best is None or key > best[0]:
            best = (key, sub)
    return np.array(best[1] if best else (), dtype=np.int64)


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(1)
    for trial in range(300):
        n = int(rng.integers(1, 11))
        dev = rng.integers(0, 4, size=n).astype(np.float32) * 0.5     # many ties
        for k in range(0, n + 1):
            got = blend.topk_hkvd(dev, k)
            want = _brute_topk(dev, k)
            assert np.array_equal(got, want), (dev, k, got, want)


def test_topk_matches_lexsort():
    rng = np.random.default_rng(2)
    for n in (1, 17, 460, 2560):
        dev = np.round(rng.random(n).astype(np.float32), 2)
        k = n // 3
        want = np.sort(np.lexsort((np.arange(n), -dev))[:k])
        assert np.array_equal(blend.topk_hkvd(dev, k), want)


def test_topk_output_sorted_and_sized():
    dev = np.array([3.0, 1.0, 3.0, 2.0, 5.0], dtype=np.float32)
    assert blend.topk_hkvd(dev, 3).tolist() == [0, 2, 4]
    assert blend.topk_hkvd(dev, 0).tolist() == []
    assert blend.topk_hkvd(dev, 9).tolist() == [0, 1, 2, 3, 4]
