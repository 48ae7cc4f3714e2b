"""Pins of the oracle's vertical-slash estimate and selection (CPU only)."""

import numpy as np
import pytest

import oracle
from oracle.estimate import estimate_rows
from tests import brute


def test_estimate_rows():
    assert estimate_rows(0, 1024, 64).tolist() == list(range(960, 1024))
    assert estimate_rows(32768, 32768, 64)[0] == 65536 - 64
    assert estimate_rows(100, 20, 64).tolist() == list(range(100, 120))


@pytest.mark.parametrize("chunk,local", [(0, 0), (8, 2)])
def test_estimate_brute_force(chunk, local):
    rng = np.random.default_rng(20)
    n, d = 36, 8
    K = rng.normal(size=(n, d))
    Q = rng.normal(size=(n, d))
    th = oracle.rope_inv_freq(d, 100.0)
    ctx = oracle.KeyContext(K, None, th, chunk, local)
    rows = estimate_rows(16, 20, 8)
    v, s = oracle.estimate_scores(Q[rows], rows, ctx, 36, 0.6)
    bv, bs = brute.estimate(Q[rows].tolist(), rows.tolist(), K.tolist(), 36,
                            brute.inv_freq(d, 100.0), 0.6)
    np.testing.assert_allclose(v, bv, atol=1e-14)
    np.testing.assert_allclose(s, bs, atol=1e-14)
    # every estimate row's probabilities sum to one
    assert v.sum() == pytest.approx(len(rows), abs=1e-12)
    assert s.sum() == pytest.approx(len(rows), abs=1e-12)


def test_estimate_ignores_dca():
    """Selection uses continuous positions (DCA on or off gives the same)."""
    rng = np.random.default_rng(21)
    n, d = 300, 16
    K, Q = rng.normal(size=(n, d)), rng.normal(size=(n, d))
    th = oracle.rope_inv_freq(d, 1e4)
    rows = estimate_rows(0, 300, 64)
    a = oracle.estimate_scores(Q[rows], rows, oracle.KeyContext(K, None, th, 64, 16), n, 0.25)
    b = oracle.estimate_scores(Q[rows], rows, oracle.KeyContext(K, None, th, 0, 0), n, 0.25)
    np.testing.assert_allclose(a[0], b[0], atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], atol=1e-14)


def test_planted_vertical_and_slash_are_found():
    """A key planted with a huge logit for every query is picked as a vertical;
    a diagonal planted at offset 5 is picked as a slash."""
    rng = np.random.default_rng(22)
    n, d = 200, 16
    K = rng.normal(size=(n, d)) * 0.1
    Q = rng.normal(size=(n, d)) * 0.1
    th = np.zeros(d // 2)            # no rotation: logits are plain q . k
    K[37] = 0
    K[37, 0] = 40.0
    Q[:, 0] += 1.0
    rows = estimate_rows(0, n, 64)
    v, s = oracle.estimate_scores(Q[rows], rows, oracle.KeyContext(K, None, th), n, 1.0)
    assert oracle.select_top(v, 1).tolist() == [37]
    K2 = rng.normal(size=(n, d)) * 0.1
    Q2 = rng.normal(size=(n, d)) * 0.1
    code = rng.normal(size=(n, d))
    for i in range(5, n):
        Q2[i] += 3 * code[i]
        K2[i - 5] += 3 * code[i]
    v2, s2 = oracle.estimate_scores(Q2[rows], rows, oracle.KeyContext(K2, None, th), n, 1.0)
    assert oracle.select_top(s2, 1).tolist() == [5]


def _brute_select(scores, k):
    order = sorted(range(len(scores)), key=lambda j: (-float(scores[j]), j))
    return sorted(order[:k])


def test_select_top_brute_force_and_ties():
    rng = np.random.default_rng(23)
    for n, k in ((10, 3), (100, 100), (100, 150), (1000, 37), (5, 0)):
        x = rng.integers(0, 5, size=n).astype(np.float32)      # many ties
        assert oracle.select_top(x, k).tolist() == _brute_select(x, min(k, n))
    x = np.array([1.0, 3.0, 3.0, 2.0, 3.0], np.float32)
    assert oracle.select_top(x, 2).tolist() == [1, 2]             # lower index wins the tie
    assert oracle.select_top(x, 3).tolist() == [1, 2, 4]
    y = rng.random(5000).astype(np.float32)
    assert oracle.select_top(y, 100).tolist() == _brute_select(y, 100)


def test_select_pattern():
    v = np.array([0.1, 0.5, 0.2, 0.5])
    s = np.array([0.9, 0.0, 0.3, 0.3])
    verts, slashes = oracle.select_pattern(v, s, 2, 3)
    assert verts.tolist() == [1, 3]
    assert slashes.tolist() == [0, 2, 3]


def test_refine_budgets():
    nv, ns, raised = oracle.refine_budgets([0.95, 0.5, 0.89, 0.2], [10, 10, 600, 1000],
                                           [20, 20, 700, 1000], 1000)
    assert raised.tolist() == [False, True, True, False]
    assert nv.tolist() == [10, 20, 1000, 1000]
    assert ns.tolist() == [20, 40, 1000, 1000]
