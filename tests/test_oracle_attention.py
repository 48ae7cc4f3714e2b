"""Pins of the oracle's dense / sparse attention and attention recall (CPU)."""

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


@pytest.mark.parametrize("chunk,local", [(0, 0), (8, 2), (12, 4)])
def test_dense_rows_brute_force(chunk, local):
    rng = np.random.default_rng(10)
    n, d = 30, 8
    ctx, K, V = _ctx(rng, n, d, chunk=chunk, local=local)
    Q = rng.normal(size=(n, d))
    freqs = brute.inv_freq(d, 100.0)
    scale = 0.37
    rows = np.arange(n)
    out, lse = oracle.dense_causal_rows(Q, rows, ctx, scale)
    for i in rows:
        o, l = brute.attention_row(Q[i].tolist(), int(i), K.tolist(), V.tolist(),
                                   list(range(i + 1)), freqs, scale, chunk, local)
        np.testing.assert_allclose(out[i], o, atol=1e-12)
        assert lse[i] == pytest.approx(l, abs=1e-12)


def test_dense_matches_textbook_sdpa():
    """No DCA: equals torch's fp64 scaled_dot_product_attention(is_causal)."""
    rng = np.random.default_rng(11)
    n, d = 64, 16
    ctx, K, V = _ctx(rng, n, d, base=1e4)
    Q = rng.normal(size=(n, d))
    th = oracle.rope_inv_freq(d, 1e4)
    h = d // 2
    def crot(x):   # rotation written with complex pairs, not via the oracle
        z = (x[:, :h] + 1j * x[:, h:]) * np.exp(1j * np.arange(n)[:, None] * th)
        return np.concatenate([z.real, z.imag], 1)
    scale = 1 / math.sqrt(d)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(crot(Q))[None, None], torch.from_numpy(crot(K))[None, None],
        torch.from_numpy(V)[None, None], is_causal=True, scale=scale)[0, 0].numpy()
    out, _ = oracle.dense_causal_rows(Q, np.arange(n), ctx, scale)
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_dca_attention_equals_causal_within_chunk():
    rng = np.random.default_rng(12)
    n, d = 256, 16
    K, V, Q = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, d))
    th = oracle.rope_inv_freq(d, 1e4)
    a = oracle.KeyContext(K, V, th, 256, 64)
    b = oracle.KeyContext(K, V, th, 0, 0)
    rows = np.array([0, 1, 100, 191, 192, 193, 255])
    oa, la = oracle.dense_causal_rows(Q[rows], rows, a, 0.25)
    ob, lb = oracle.dense_causal_rows(Q[rows], rows, b, 0.25)
    np.testing.assert_allclose(oa, ob, atol=1e-11)
    np.testing.assert_allclose(la, lb, atol=1e-11)
    # and beyond C it does differ
    rows2 = np.array([255])
    K2, V2 = rng.normal(size=(600, d)), rng.normal(size=(600, d))
    q2 = rng.normal(size=(1, d))
    c = oracle.KeyContext(K2, V2, th, 256, 64)
    e = oracle.KeyContext(K2, V2, th, 0, 0)
    _, l1 = oracle.dense_causal_rows(q2, np.array([599]), c, 0.25)
    _, l2 = oracle.dense_causal_rows(q2, np.array([599]), e, 0.25)
    assert abs(l1[0] - l2[0]) > 1e-6


def test_critical_set_semantics():
    verts = np.array([0, 3, 7, 20])
    slashes = np.array([0, 2, 4, 30])
    assert oracle.critical_set(6, verts, slashes).tolist() == [0, 2, 3, 4, 6]
    assert oracle.critical_set(7, verts, slashes).tolist() == [0, 3, 5, 7]
    assert oracle.critical_set(0, np.array([5]), np.array([1])).tolist() == []


def test_critical_pair_total_counts_the_sets():
    """The pair total the full-size GPU tests hold the kernel's pair count
    to equals the sum of |C_i| over the oracle's critical sets, with
    verticals on slash diagonals (overlaps), indices past the chunk and a
    chunk that starts inside the context."""
    from tests.gpu_util import critical_pair_total
    rng = np.random.default_rng(11)
    for c0, c1 in [(0, 300), (200, 520), (513, 514)]:
        verts = np.sort(rng.choice(c1 + 40, size=45, replace=False))
        slashes = np.sort(rng.choice(c1 + 40, size=70, replace=False))
        # plant overlaps: vertical v on the diagonal o of row v + o
        verts = np.unique(np.concatenate([verts, [c0 - slashes[3]] if c0 > slashes[3] else []])
                          .astype(np.int64))
        want = sum(oracle.critical_set(i, verts, slashes).size for i in range(c0, c1))
        assert critical_pair_total(verts, slashes, c0, c1) == want


@pytest.mark.parametrize("chunk,local", [(0, 0), (8, 2)])
def test_sparse_rows_brute_force(chunk, local):
    rng = np.random.default_rng(13)
    n, d = 40, 8
    ctx, K, V = _ctx(rng, n, d, chunk=chunk, local=local)
    Q = rng.normal(size=(n, d))
    verts = np.array([0, 1, 9, 17, 33])
    slashes = np.array([0, 1, 5, 8, 16, 35])
    freqs = brute.inv_freq(d, 100.0)
    rows = np.arange(n)
    out, lse, sizes = oracle.sparse_rows(Q, rows, ctx, verts, slashes, 0.5)
    for i in rows:
        keys = sorted(set(int(v) for v in verts if v <= i) |
                      set(int(i - o) for o in slashes if o <= i))
        assert sizes[i] == len(keys)
        o, l = brute.attention_row(Q[i].tolist(), int(i), K.tolist(), V.tolist(),
                                   keys, freqs, 0.5, chunk, local)
        np.testing.assert_allclose(out[i], o, atol=1e-12)
        assert lse[i] == pytest.approx(l, abs=1e-12)


def test_sparse_all_verticals_is_dense():
    rng = np.random.default_rng(14)
    n, d = 50, 8
    ctx, _, _ = _ctx(rng, n, d, chunk=16, local=4)
    Q = rng.normal(size=(n, d))
    rows = np.arange(n)
    od, ld = oracle.dense_causal_rows(Q, rows, ctx, 0.3)
    os_, ls, _ = oracle.sparse_rows(Q, rows, ctx, np.arange(n), np.array([], np.int64), 0.3)
    np.testing.assert_allclose(os_, od, atol=1e-13)
    np.testing.assert_allclose(ls, ld, atol=1e-13)


def test_sparse_slash_band_is_sliding_window():
    """Slashes {0..w-1} and no verticals = textbook sliding-window attention."""
    rng = np.random.default_rng(15)
    n, d, w = 48, 16, 5
    ctx, K, V = _ctx(rng, n, d, base=1e4)
    Q = rng.normal(size=(n, d))
    th = oracle.rope_inv_freq(d, 1e4)
    h = d // 2
    def crot(x):
        z = (x[:, :h] + 1j * x[:, h:]) * np.exp(1j * np.arange(n)[:, None] * th)
        return np.concatenate([z.real, z.imag], 1)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    mask = torch.from_numpy((j <= i) & (i - j < w))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(crot(Q))[None, None], torch.from_numpy(crot(K))[None, None],
        torch.from_numpy(V)[None, None], attn_mask=mask[None, None], scale=0.25)[0, 0].numpy()
    out, _, _ = oracle.sparse_rows(Q, np.arange(n), ctx, np.array([], np.int64), np.arange(w), 0.25)
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_sparse_single_key_and_empty():
    rng = np.random.default_rng(16)
    n, d = 20, 8
    ctx, K, V = _ctx(rng, n, d)
    Q = rng.normal(size=(n, d))
    out, lse, _ = oracle.sparse_rows(Q, np.arange(n), ctx, np.array([], np.int64), np.array([0]), 1.0)
    np.testing.assert_allclose(out, V, atol=1e-14)
    # logit of the diagonal pair: relative position 0, so plain q . k
    np.testing.assert_allclose(lse, np.sum(Q * K, 1), atol=1e-12)
    out, lse, sizes = oracle.sparse_rows(Q[:3], np.arange(3), ctx, np.array([10]), np.array([5]), 1.0)
    assert np.all(out == 0) and np.all(np.isneginf(lse)) and np.all(sizes == 0)


def test_recall_properties():
    rng = np.random.default_rng(17)
    n, d = 60, 8
    ctx, _, _ = _ctx(rng, n, d, chunk=16, local=4)
    Q = rng.normal(size=(n, d)) * 2
    rows = np.arange(10, n)
    full, sp, rec = oracle.attention_recall(Q[rows], rows, ctx, np.arange(n), np.array([], np.int64), 0.5)
    np.testing.assert_allclose(rec, 1.0, atol=1e-14)
    v1, s1 = np.array([0, 7]), np.array([0, 1])
    v2, s2 = np.array([0, 3, 7, 30]), np.array([0, 1, 2, 9])
    _, _, r1 = oracle.attention_recall(Q[rows], rows, ctx, v1, s1, 0.5)
    _, _, r2 = oracle.attention_recall(Q[rows], rows, ctx, v2, s2, 0.5)
    assert np.all((r1 > 0) & (r1 <= 1)) and np.all(r2 >= r1 - 1e-15)
    # recall = mass of the dense softmax on the critical set
    for a, i in enumerate(rows):
        lg = oracle.attention_logits(Q[i], i, ctx, np.arange(i + 1), 0.5)
        p = np.exp(lg - lg.max())
        p /= p.sum()
        cs = oracle.critical_set(i, v1, s1)
        assert r1[a] == pytest.approx(p[cs].sum(), rel=1e-12)
    assert np.all(full >= sp)


@pytest.mark.parametrize("mode,bits", [("bf16", 8), ("fp16", 11)])
@pytest.mark.parametrize("chunk,local", [(0, 0), (12, 4)])
def test_rounded_operands(chunk, local, mode, bits):
    """operands="bf16" / "fp16": the cached keys are the roundings of the
    exact rotated keys (representable, within half an ulp of a `bits`-bit
    significand); continuous-position keys rotate back to the pre-RoPE keys
    within that rounding; with the rotation switched off and bf16 inputs the
    rounding is a no-op, so both modes agree exactly (nothing else is
    rounded); with it on they differ by no more than the operand rounding
    allows."""
    rnd = {"bf16": oracle.bf16_round64, "fp16": oracle.fp16_round64}[mode]
    rng = np.random.default_rng(21)
    n, d = 40, 8
    K = oracle.bf16_round(rng.normal(size=(n, d))).astype(np.float64)
    V = rng.normal(size=(n, d))
    Q = oracle.bf16_round(rng.normal(size=(n, d))).astype(np.float64)
    th = oracle.rope_inv_freq(d, 100.0)
    exact = oracle.KeyContext(K, V, th, chunk, local)
    rc = oracle.KeyContext(K, V, th, chunk, local, operands=mode)
    kd, ke = rc.k_dca(), exact.k_dca()
    assert np.array_equal(rnd(kd), kd)
    assert np.all(np.abs(kd - ke) <= np.ldexp(1.0, np.frexp(ke)[1] - bits - 1))
    back = oracle.rope_rotate(rc.k_cont(), -np.arange(n), th)
    assert np.max(np.abs(back - K)) <= 2.0 ** -(bits - 1) * np.max(np.abs(K))
    if chunk == 0:
        assert np.array_equal(rc.k_cont(), kd)
    rows = np.arange(n)
    oe, le = oracle.dense_causal_rows(Q, rows, exact, 0.4)
    ob, lb = oracle.dense_causal_rows(Q, rows, rc, 0.4)
    # logits move by at most 2 * 2^-bits * sm |q| |k| (both operands rounded)
    bound = 2 * 2.0 ** -bits * 0.4 * np.linalg.norm(Q, axis=1) * np.max(np.linalg.norm(K, axis=1))
    assert np.max(np.abs(oe - ob)) > 0 and np.all(np.abs(le - lb) <= bound)
    zero = np.zeros(d // 2)
    a = oracle.KeyContext(K, V, zero, chunk, local)
    b = oracle.KeyContext(K, V, zero, chunk, local, operands=mode)
    oa, la = oracle.sparse_rows(Q, rows, a, [0, 3], [0, 1, 5], 0.4)[:2]
    ob2, lb2 = oracle.sparse_rows(Q, rows, b, [0, 3], [0, 1, 5], 0.4)[:2]
    assert np.array_equal(oa, ob2) and np.array_equal(la, lb2)
    with pytest.raises(ValueError):
        oracle.KeyContext(K, V, th, operands="fp8")


def test_fp16_round64_library():
    """Direct fp64 -> fp16 rounding: torch's float32 -> float16 conversion on
    float32-representable values, ties to even, and no double rounding just
    off a tie."""
    rng = np.random.default_rng(8)
    x = (rng.normal(size=10000) * 10.0 ** rng.integers(-3, 4, 10000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.fp16_round64(x.astype(np.float64)), ref)
    assert oracle.fp16_round64(np.array([1 + 2 ** -11]))[0] == 1.0            # tie -> even
    assert oracle.fp16_round64(np.array([1 + 3 * 2 ** -11]))[0] == 1 + 2 ** -9  # tie -> even
    assert oracle.fp16_round64(np.array([1 + 2 ** -11 + 2 ** -40]))[0] == 1 + 2 ** -10
