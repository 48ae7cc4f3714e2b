"""Pins of the oracle's fixed (A-shape) pattern and the per-head candidate
choice (CPU)."""

from collections import deque

import numpy as np
import pytest
import torch

import oracle


def _streaming_cache_keys(n, n_sink, n_local):
    """Keys held by a streaming KV cache that keeps the first n_sink tokens
    and a first-in first-out window of the latest n_local tokens, as each
    token is appended: the operational form of the sink + window rule."""
    sinks, window, held = [], deque(maxlen=n_local if n_local > 0 else None), []
    for i in range(n):
        if i < n_sink:
            sinks.append(i)
        elif n_local > 0:
            window.append(i)
        # a token in both roles (i < n_sink and recent) is held once
        recent = [j for j in range(max(0, i - n_local + 1), i + 1)] if n_local > 0 else []
        held.append(sorted(set(sinks) | set(window) | set(recent)))
    return held


@pytest.mark.parametrize("n_sink,n_local", [(0, 1), (0, 5), (3, 4), (4, 0), (40, 3), (2, 60),
                                            (0, 0)])
def test_a_shape_set_is_the_streaming_cache(n_sink, n_local):
    n = 37
    held = _streaming_cache_keys(n, n_sink, n_local)
    for i in range(n):
        assert oracle.a_shape_set(i, n_sink, n_local).tolist() == held[i], i


@pytest.mark.parametrize("n_sink,n_local", [(0, 1), (3, 4), (4, 0), (40, 3), (2, 60), (7, 7)])
def test_a_shape_lists_encode_the_set(n_sink, n_local):
    """The vertical/slash encoding gives the same set through the
    vertical-slash critical-set rule, row by row."""
    n = 41
    verts, slashes = oracle.a_shape_lists(n_sink, n_local, n)
    assert verts.size == min(n_sink, n) and slashes.size == min(n_local, n)
    for i in range(n):
        np.testing.assert_array_equal(oracle.critical_set(i, verts, slashes),
                                      oracle.a_shape_set(i, n_sink, n_local))


def _ctx(rng, n, d):
    K = rng.normal(size=(n, d))
    V = rng.normal(size=(n, d))
    return oracle.KeyContext(K, V, oracle.rope_inv_freq(d, 1e4)), K, V


def test_sliding_window_attention_is_masked_sdpa():
    """n_sink = 0: the A-shape is a causal band of width w, which torch's fp64
    scaled_dot_product_attention computes with an explicit boolean mask."""
    rng = np.random.default_rng(31)
    n, d, w = 48, 16, 9
    ctx, K, V = _ctx(rng, n, d)
    Q = rng.normal(size=(n, d))
    scale = 0.3
    verts, slashes = oracle.a_shape_lists(0, w, n)
    out, _, sizes = oracle.sparse_rows(Q, np.arange(n), ctx, verts, slashes, scale)
    pos = np.arange(n)
    qr = oracle.rope_apply(Q[None], pos, ctx.inv_freq)[0]
    kr = oracle.rope_apply(K[None], pos, ctx.inv_freq)[0]
    i, j = np.meshgrid(pos, pos, indexing="ij")
    mask = torch.from_numpy((j <= i) & (i - j < w))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qr)[None], torch.from_numpy(kr)[None], torch.from_numpy(V)[None],
        attn_mask=mask[None], scale=scale)[0].numpy()
    np.testing.assert_allclose(out, ref, atol=1e-12)
    np.testing.assert_array_equal(sizes, np.minimum(pos + 1, w))


def test_a_shape_wide_window_is_dense():
    rng = np.random.default_rng(32)
    n, d = 40, 8
    ctx, _, _ = _ctx(rng, n, d)
    Q = rng.normal(size=(n, d))
    rows = np.arange(n)
    verts, slashes = oracle.a_shape_lists(3, n, n)
    out, lse, _ = oracle.sparse_rows(Q, rows, ctx, verts, slashes, 0.5)
    ref, ref_lse = oracle.dense_causal_rows(Q, rows, ctx, 0.5)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12)


def test_choose_candidates_argmax_first_on_ties():
    scores = np.array([[0.50, 0.90, 0.70, 0.20],
                       [0.60, 0.90, 0.95, 0.20],
                       [0.60, 0.80, 0.95, 0.10]])
    # head 0: tie 0.60 between candidates 1 and 2 -> 1; head 1: tie of 0 and 1
    # -> 0; head 2: 1 beats 0, ties with 2 -> 1; head 3: 0
    np.testing.assert_array_equal(oracle.choose_candidates(scores), [1, 0, 1, 0])


def test_choose_candidates_nested_budgets():
    """Nested candidates (each set contains the previous one) have
    non-decreasing recall; the choice is the first candidate that reaches the
    largest recall."""
    rng = np.random.default_rng(33)
    n, d = 64, 8
    ctx, _, _ = _ctx(rng, n, d)
    Q = rng.normal(size=(n, d))
    rows = np.arange(32, n)
    cands = [(2, 4), (4, 8), (8, 16), (64, 64)]
    rec = []
    for s_, w_ in cands:
        v, sl = oracle.a_shape_lists(s_, w_, n)
        rec.append(oracle.attention_recall(Q[rows], rows, ctx, v, sl, 0.4)[2].mean())
    assert all(b >= a - 1e-15 for a, b in zip(rec, rec[1:]))
    assert rec[-1] == pytest.approx(1.0, abs=1e-14)
    choice = oracle.choose_candidates(np.array(rec)[:, None])[0]
    assert rec[choice] == max(rec) and all(r < max(rec) for r in rec[:choice])


def test_refine_sizes_hand_cases():
    """One refinement round over mixed kinds (threshold 0.9, 1000 keys =
    16 key blocks): low heads double their own size, capped; others stay."""
    kinds = ["vs", "vs", "block", "block", "a_shape", "a_shape", "vs"]
    sizes = [(10, 20), (10, 20), (3,), (10,), (4, 300), (4, 1000), (1000, 1000)]
    rec = [0.5, 0.95, 0.2, 0.3, 0.1, 0.1, 0.1]
    new, raised = oracle.refine_sizes(rec, kinds, sizes, 1000)
    assert new == [(20, 40), (10, 20), (6,), (16,), (4, 600), (4, 1000), (1000, 1000)]
    assert raised.tolist() == [True, False, True, True, True, False, False]
    # the vertical-slash rule is the existing one
    nv, ns, r2 = oracle.refine_budgets(rec[:2], [10, 10], [20, 20], 1000)
    assert [tuple(x) for x in zip(nv, ns)] == new[:2] and r2.tolist() == raised[:2].tolist()
