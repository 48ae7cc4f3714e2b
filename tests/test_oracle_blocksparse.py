"""Pins of the oracle's block-sparse pattern (CPU): block scores against the
brute-force continuous-position logits averaged over each block pair, the
selection rule against a sort, and the attention against dense attention,
block-local masked SDPA and brute-force rows with DCA."""

import math

import numpy as np
import pytest
import torch

import oracle
from tests import brute


def _ctx(rng, n, d, base=100.0, chunk=0, local=0):
    K = rng.normal(size=(n, d))
    V = rng.normal(size=(n, d))
    return oracle.KeyContext(K, V, oracle.rope_inv_freq(d, base), chunk, local), K, V


@pytest.mark.parametrize("c0,n,chunk,local", [(128, 72, 0, 0), (0, 150, 0, 0),
                                              (192, 64, 128, 32)])
def test_block_scores_are_mean_block_logits(c0, n, chunk, local):
    """By bilinearity a block score is the mean of the continuous-position
    logits over the block pair; those come from complex-pair brute force
    (relative position i - j), partial blocks included."""
    rng = np.random.default_rng(40)
    d, scale = 8, 0.3
    c1 = c0 + n
    ctx, K, _ = _ctx(rng, c1, d, chunk=chunk, local=local)
    Q = rng.normal(size=(n, d))
    s = oracle.block_scores(Q, c0, ctx, scale)
    freqs = brute.inv_freq(d, 100.0)
    B = oracle.BLOCK
    n_qb, n_kb = -(-n // B), -(-c1 // B)
    assert s.shape == (n_qb, n_kb)
    for qb in range(n_qb):
        diag = c0 // B + qb
        qi = range(c0 + qb * B, min(c0 + (qb + 1) * B, c1))
        for kb in range(n_kb):
            if kb > diag:
                assert s[qb, kb] == -math.inf
                continue
            kj = range(kb * B, min((kb + 1) * B, c1))
            terms = [scale * brute.rope_dot(Q[i - c0].tolist(), K[j].tolist(), i - j, freqs)
                     for i in qi for j in kj]
            assert s[qb, kb] == pytest.approx(math.fsum(terms) / len(terms), abs=1e-12)


def test_select_blocks_rule():
    sc = np.array([0.5, 0.9, 0.9, 0.1, 0.7, 0.9, 2.0])
    # diag 6 (score ignored); ties at 0.9 go to the lower index
    np.testing.assert_array_equal(oracle.select_blocks(sc, 6, 3), [1, 2, 6])
    np.testing.assert_array_equal(oracle.select_blocks(sc, 6, 4), [1, 2, 5, 6])
    np.testing.assert_array_equal(oracle.select_blocks(sc, 6, 1), [6])
    np.testing.assert_array_equal(oracle.select_blocks(sc, 6, 0), [6])
    np.testing.assert_array_equal(oracle.select_blocks(sc, 6, 99), np.arange(7))
    np.testing.assert_array_equal(oracle.select_blocks(sc, 0, 5), [0])
    rng = np.random.default_rng(41)
    x = rng.normal(size=300)
    for k in (1, 2, 17, 150):
        order = np.argsort(-x[:200], kind="stable")[:k - 1]
        np.testing.assert_array_equal(oracle.select_blocks(x, 200, k),
                                      np.sort(np.append(order, 200)))


def test_all_blocks_is_dense():
    rng = np.random.default_rng(42)
    n, d = 200, 8
    ctx, _, _ = _ctx(rng, n, d, chunk=96, local=32)
    Q = rng.normal(size=(n, d))
    rows = np.arange(n)
    out, lse, sizes = oracle.block_sparse_rows(
        Q, rows, ctx, lambda i: np.arange(i // oracle.BLOCK + 1), 0.4)
    ref, ref_lse = oracle.dense_causal_rows(Q, rows, ctx, 0.4)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12)
    np.testing.assert_array_equal(sizes, rows + 1)


def test_diagonal_block_only_is_block_local_sdpa():
    """Only the diagonal block (no DCA): causal attention inside each 64-row
    block, which torch's fp64 SDPA computes with a block-diagonal mask."""
    rng = np.random.default_rng(43)
    n, d = 160, 16
    ctx, K, V = _ctx(rng, n, d, base=1e4)
    Q = rng.normal(size=(n, d))
    rows = np.arange(n)
    out, _, _ = oracle.block_sparse_rows(Q, rows, ctx, lambda i: [i // oracle.BLOCK], 0.25)
    qr = oracle.rope_apply(Q[None], rows, ctx.inv_freq)[0]
    kr = oracle.rope_apply(K[None], rows, ctx.inv_freq)[0]
    i, j = np.meshgrid(rows, rows, indexing="ij")
    mask = torch.from_numpy((j <= i) & (j // 64 == i // 64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qr)[None], torch.from_numpy(kr)[None], torch.from_numpy(V)[None],
        attn_mask=mask[None], scale=0.25)[0].numpy()
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_block_rows_brute_force_dca():
    rng = np.random.default_rng(44)
    n, d, chunk, local = 260, 8, 128, 32
    ctx, K, V = _ctx(rng, n, d, chunk=chunk, local=local)
    Q = rng.normal(size=(n, d))
    kept = {0: [0], 1: [0, 1], 2: [1, 2], 3: [0, 2, 3], 4: [3, 4]}
    rows = np.array([0, 63, 64, 100, 128, 191, 200, 255, 256, 259])
    out, lse, sizes = oracle.block_sparse_rows(Q[rows], rows, ctx,
                                               lambda i: kept[i // 64], 0.35)
    freqs = brute.inv_freq(d, 100.0)
    for a, i in enumerate(rows):
        js = [j for b in kept[i // 64] for j in range(64 * b, 64 * b + 64) if j <= i]
        assert sizes[a] == len(js)
        o, l = brute.attention_row(Q[i].tolist(), int(i), K.tolist(), V.tolist(), js, freqs,
                                   0.35, chunk, local)
        np.testing.assert_allclose(out[a], o, atol=1e-12)
        assert lse[a] == pytest.approx(l, abs=1e-12)
