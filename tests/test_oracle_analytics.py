"""Pins of the oracle's deviation analytics (CPU).

* Spearman: equals scipy's spearmanr (a library routine of the same
  definition) on random data with ties; +1 for any increasing transform, -1
  for a decreasing one; tied ranks share their mean rank.
* Attention matrix: rows are probability vectors with zeros past each row's
  last key; a single key gets probability 1; equal scores give a uniform
  row; with one KV head per query head it matches a direct softmax written
  per row; GQA reads KV head h // group.
* Attention deviation: 0 for equal matrices, the Frobenius norm of a known
  difference, symmetric.
* Top share: closed forms on small arrays (all equal -> frac; one nonzero ->
  1)."""
import math

import numpy as np
import pytest
from scipy import stats

from oracle import analytics as A


def test_spearman_matches_scipy_with_ties():
    rng = np.random.default_rng(0)
    for n in (2, 5, 17, 300):
        x = rng.integers(0, 7, n).astype(float)     # many ties
        y = x + rng.normal(0, 2, n)
        assert abs(A.spearman(x, y) - stats.spearmanr(x, y).statistic) < 1e-12
        y2 = rng.integers(0, 3, n).astype(float)
        if np.ptp(y2) > 0 and np.ptp(x) > 0:
            assert abs(A.spearman(x, y2) - stats.spearmanr(x, y2).statistic) < 1e-12


def test_spearman_monotone_transforms():
    x = np.array([3.0, -1.0, 2.5, 10.0, 0.0])
    assert A.spearman(x, np.exp(x)) == pytest.approx(1.0)
    assert A.spearman(x, -x ** 3) == pytest.approx(-1.0)
    assert np.array_equal(A.ranks(np.array([5.0, 1.0, 5.0, 2.0])), [3.5, 1.0, 3.5, 2.0])


def test_attention_matrix_rows_and_masks():
    rng = np.random.default_rng(1)
    q = rng.normal(size=(3, 4, 8))
    k = rng.normal(size=(6, 2, 8))
    last = [0, 3, 5]
    P = A.attention_matrix(q, k, last)
    for i, L in enumerate(last):
        assert np.allclose(P[i, :, :L + 1].sum(-1), 1.0)
        assert np.all(P[i, :, L + 1:] == 0)
    assert np.all(P[0, :, 0] == 1.0)                     # one key
    # GQA: query head h reads KV head h // 2; against a direct per-row softmax
    for i, L in enumerate(last):
        for h in range(4):
            s = np.array([q[i, h] @ k[t, h // 2] for t in range(L + 1)]) / math.sqrt(8)
            p = np.exp(s - s.max())
            assert np.allclose(P[i, h, :L + 1], p / p.sum(), atol=1e-15)
    # equal scores: uniform
    P2 = A.attention_matrix(np.zeros((1, 2, 8)), k, [4])
    assert np.allclose(P2[0, :, :5], 0.2)


def test_attention_deviation_norm():
    a = np.zeros((1, 2, 3))
    b = a.copy()
    assert A.attention_deviation(a, b) == 0.0
    b[0, 1, 2] = 0.3
    b[0, 0, 0] = -0.4
    assert A.attention_deviation(a, b) == pytest.approx(0.5)
    assert A.attention_deviation(b, a) == pytest.approx(0.5)


def test_top_share_closed_forms():
    assert A.top_share(np.ones(20), 0.15) == pytest.approx(3 / 20)    # ceil(0.15 * 20) = 3
    d = np.zeros(10)
    d[7] = 2.0
    assert A.top_share(d, 0.1) == 1.0
    assert A.top_share(np.array([4.0, 3.0, 2.0, 1.0]), 0.5) == pytest.approx(0.7)
