"""GPU parity of the fixed head patterns and the per-head pattern search,
through the C ABI, against the fp64 oracle: the A-shape fill (bit-exact, and
rows of other heads untouched), one layer mixing A-shape and vertical-slash
heads (every row of the last chunk, exact pair counts), and the search's
recall scores and choices."""

import time

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import FOURTEEN_B_512K_REFINE, SEVEN_B_128K, scaled
from tests.gpu_util import (DEV, build_cache, compare, dca_of, host64, lse_compare,
                            oracle_freqs, oracle_inputs, product_sm, rope_of)

pytestmark = pytest.mark.gpu

L = pytest.importorskip("long_context_sparse_rope_amd")

# 7B grouping at D 128 with DCA (period S = 768), four 1024-token chunks
CFG = scaled(SEVEN_B_128K, n_heads=14, n_kv_heads=2, seq_len=4096, prefill_chunk=1024,
             dca_chunk=1024, dca_local=256, n_vert=64, n_slash=128)

# the refinement-stress planting (far sinks, per-head stripes) at the same
# small shape: the A-shape candidates cover little of it
CFG_STRIPES = scaled(FOURTEEN_B_512K_REFINE, n_heads=10, n_kv_heads=2, seq_len=4096,
                     prefill_chunk=1024, dca_chunk=1024, dca_local=256, n_vert=64,
                     n_slash=128)

VS = lambda nv, ns: {"kind": "vs", "n_vert": nv, "n_slash": ns}          # noqa: E731
AS = lambda s, w: {"kind": "a_shape", "n_sink": s, "n_local": w}          # noqa: E731
BS = lambda k: {"kind": "block", "n_blocks": k}                           # noqa: E731


def _layer(cfg):
    return L.ChunkedSparsePrefill(cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len,
                                  rope_of(cfg), dca_of(cfg),
                                  product_sm(cfg),
                                  cfg.n_vert, cfg.n_slash, cfg.last_q, DEV)


def _contexts(cfg, k, v, upto):
    _, ko, vo = oracle_inputs(k[:1], k, v)
    th = oracle_freqs(cfg)
    return [oracle.KeyContext(ko[g, :upto], vo[g, :upto], th, cfg.dca_chunk, cfg.dca_local) for g in range(cfg.n_kv_heads)]


@pytest.mark.parametrize("n_sink,n_local,n_ctx", [(16, 2048, 65536), (0, 300, 1000),
                                                  (50, 0, 40), (64, 4096, 1000), (3, 5, 0),
                                                  (80, 4100, 1 << 20)])
def test_fill_a_shape_bit_exact(n_sink, n_local, n_ctx):
    print(f"[fill] sink {n_sink} local {n_local} n_ctx {n_ctx}", flush=True)
    H, mv, ms = 6, 80, 4100
    pat = L.Pattern(H, mv, ms, DEV)
    pat.vert_idx.fill_(7)
    pat.slash_idx.fill_(9)
    pat.vert_cnt.fill_(3)
    pat.slash_cnt.fill_(4)
    mask = [1, 0, 1, 1, 0, 1]
    L.pattern_fill_a_shape(pat, n_sink, n_local, n_ctx, head_mask=mask)
    torch.cuda.synchronize()
    v_ref, s_ref = oracle.a_shape_lists(n_sink, n_local, n_ctx)
    vi, si = pat.vert_idx.cpu().numpy(), pat.slash_idx.cpu().numpy()
    vc, sc = pat.vert_cnt.cpu().numpy(), pat.slash_cnt.cpu().numpy()
    for h in range(H):
        if mask[h]:
            ev = np.full(mv, -1)
            ev[:v_ref.size] = v_ref
            es = np.full(ms, -1)
            es[:s_ref.size] = s_ref
            np.testing.assert_array_equal(vi[h], ev)
            np.testing.assert_array_equal(si[h], es)
            assert vc[h] == v_ref.size and sc[h] == s_ref.size
        else:
            assert np.all(vi[h] == 7) and np.all(si[h] == 9) and vc[h] == 3 and sc[h] == 4


def test_mixed_head_patterns_layer():
    """Heads cycle through a vertical-slash estimate, two A-shapes, a pure
    sliding window, sinks only and two block-sparse budgets; the whole chunk
    loop runs, then every row of the last chunk is checked against the oracle
    (A-shape heads on the oracle's own lists, vertical-slash and block heads
    on the GPU's selection)."""
    cfg = CFG
    q, k, v = synth.generate(cfg, DEV)
    layer = _layer(cfg)
    kinds = [VS(64, 128), AS(16, 256), BS(4), AS(0, 100), AS(64, 0), BS(11), AS(4, 700),
             VS(32, 200)]
    configs = [kinds[h % len(kinds)] for h in range(cfg.n_heads)]
    layer.set_head_patterns(configs)
    N, C = cfg.seq_len, cfg.prefill_chunk
    out = torch.empty(cfg.n_heads, N, cfg.head_dim, device=DEV)
    lse = torch.empty(cfg.n_heads, N, device=DEV)
    layer.run(q, k, v, C, out=out, lse=lse)
    c0 = N - C
    stats = torch.zeros(2, dtype=torch.int64, device=DEV)
    layer.attend(q[:, c0:], c0, stats=stats)
    torch.cuda.synchronize()
    verts, slashes = layer.pattern.lists()
    bidx, bcnt = layer.block_pattern.idx.cpu().numpy(), layer.block_pattern.cnt.cpu().numpy()
    qo, _, _ = oracle_inputs(q, k[:1], v[:1])
    ctxs = _contexts(cfg, k, v, N)
    rows = np.arange(c0, N)
    G = cfg.n_heads // cfg.n_kv_heads
    pairs = 0
    for h, c in enumerate(configs):
        if c["kind"] == "block":
            assert np.all(bcnt[h] == np.minimum(c["n_blocks"], c0 // 64 + np.arange(16) + 1))
            kept = lambda i, h=h: bidx[h, (i - c0) // 64, :bcnt[h, (i - c0) // 64]]  # noqa
            ro, rl, sizes = oracle.block_sparse_rows(qo[h, rows], rows, ctxs[h // G], kept,
                                                     layer.sm_scale)
        else:
            if c["kind"] == "a_shape":
                ov, os_ = oracle.a_shape_lists(c["n_sink"], c["n_local"], N)
                np.testing.assert_array_equal(verts[h].numpy(), ov)
                np.testing.assert_array_equal(slashes[h].numpy(), os_)
            else:
                ov, os_ = verts[h].numpy(), slashes[h].numpy()
                assert ov.size == min(c["n_vert"], N) and os_.size == min(c["n_slash"], N)
            ro, rl, sizes = oracle.sparse_rows(qo[h, rows], rows, ctxs[h // G], ov, os_,
                                               layer.sm_scale)
        print(f"[mixed] head {h} {c}", flush=True)
        compare(host64(out[h, c0:]), ro)
        lse_compare(host64(lse[h, c0:]), rl)
        pairs += int(sizes.sum())
    assert int(stats[1].item()) == pairs


@pytest.mark.parametrize("cfg", [CFG, CFG_STRIPES], ids=["sinks_band", "stripes"])
def test_search_head_patterns(cfg):
    """Candidates scored by mean attention recall over the sampled rows of two
    calibration chunks; GPU scores against the oracle's recall on the same
    sets, and each head's choice by the rule."""
    q, k, v = synth.generate(cfg, DEV)
    layer = _layer(cfg)
    build_cache(layer, k, v, cfg.seq_len)
    cands = [AS(16, 128), VS(32, 96), BS(4), AS(64, 512), VS(128, 384), BS(8)]
    chunks = [(2048, 1024), (3072, 1024)]
    rng = np.random.default_rng(7)
    off = np.unique(np.concatenate([np.arange(1024 - 64, 1024), rng.integers(0, 1024, 32)]))
    rows = torch.tensor(off, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    choice, scores = L.search_head_patterns(layer, q, chunks, cands, rows)
    torch.cuda.synchronize()
    print(f"[search] {len(cands)} candidates x {len(chunks)} chunks: "
          f"{(time.perf_counter() - t0) * 1e3:.1f} ms", flush=True)
    # the layer's own configuration is restored
    assert layer.a_shape == [None] * cfg.n_heads and layer.blocks == [None] * cfg.n_heads
    assert layer.n_vert == [cfg.n_vert] * cfg.n_heads
    qo, _, _ = oracle_inputs(q, k[:1], v[:1])
    ctxs = _contexts(cfg, k, v, cfg.seq_len)
    G = cfg.n_heads // cfg.n_kv_heads
    ref = np.zeros((len(cands), cfg.n_heads))
    for ci, c in enumerate(cands):
        layer.set_head_patterns([c] * cfg.n_heads)
        for c0, n in chunks:
            layer.estimate(q[:, c0:c0 + n], c0)
            verts, slashes = layer.pattern.lists()
            r = c0 + off
            for h in range(cfg.n_heads):
                if c["kind"] == "block":
                    bidx = layer.block_pattern.idx[h].cpu().numpy()
                    bcnt = layer.block_pattern.cnt[h].cpu().numpy()
                    kept = lambda i, c0=c0: bidx[(i - c0) // 64, :bcnt[(i - c0) // 64]]  # noqa
                    _, sl, _ = oracle.block_sparse_rows(qo[h, r], r, ctxs[h // G], kept,
                                                        layer.sm_scale)
                    _, fl = oracle.dense_causal_rows(qo[h, r], r, ctxs[h // G], layer.sm_scale)
                    rec = np.exp(sl - fl)
                else:
                    if c["kind"] == "a_shape":
                        ov, os_ = oracle.a_shape_lists(c["n_sink"], c["n_local"], c0 + n)
                    else:
                        ov, os_ = verts[h].numpy(), slashes[h].numpy()
                    rec = oracle.attention_recall(qo[h, r], r, ctxs[h // G], ov, os_,
                                                  layer.sm_scale)[2]
                ref[ci, h] += rec.mean() / len(chunks)
    got = np.asarray(scores)
    d = np.abs(got - ref)
    print(f"[search] {cfg.name}: score max diff {d.max():.2e}; choices {choice}", flush=True)
    print("[search] scores (candidate x head):\n" + np.array2string(got, precision=3), flush=True)
    assert d.max() <= 5e-3
    # the rule on the GPU's own scores, exactly
    np.testing.assert_array_equal(choice, oracle.choose_candidates(got))
    # against the oracle's scores: equal choice wherever the oracle's best
    # candidate leads the others by more than the score tolerance
    best = oracle.choose_candidates(ref)
    for h in range(cfg.n_heads):
        others = np.delete(ref[:, h], best[h])
        if ref[best[h], h] - others.max() > 1e-2:
            assert choice[h] == best[h], h
        else:
            assert ref[choice[h], h] >= ref[best[h], h] - 1e-2, h


def test_refinement_over_mixed_kinds():
    """Refinement on the stripes layer with vertical-slash, block-sparse and
    A-shape heads at small sizes: every round's decisions are the oracle's
    rule applied to the GPU's recall, raised heads do not lose recall (their
    sets are nested), and the final rows match the oracle on the final
    patterns."""
    cfg = CFG_STRIPES
    q, k, v = synth.generate(cfg, DEV)
    layer = _layer(cfg)
    build_cache(layer, k, v, cfg.seq_len)
    kinds = [VS(8, 16), BS(2), AS(4, 64), VS(32, 8), BS(1)]
    configs = [kinds[h % len(kinds)] for h in range(cfg.n_heads)]
    layer.set_head_patterns(configs)
    c0, c1 = 3072, 4096
    qc = q[:, c0:c1]
    out = torch.empty(cfg.n_heads, c1 - c0, cfg.head_dim, device=DEV)
    lse = torch.empty(cfg.n_heads, c1 - c0, device=DEV)
    layer.estimate(qc, c0)
    layer.attend(qc, c0, out=out, lse=lse)
    rng = np.random.default_rng(11)
    off = np.unique(np.concatenate([np.arange(1024 - 64, 1024), rng.integers(0, 1024, 32)]))
    rows = torch.tensor(off, dtype=torch.int32, device=DEV)

    def sizes():
        res = []
        for h in range(cfg.n_heads):
            if layer.blocks[h] is not None:
                res.append((layer.blocks[h],))
            elif layer.a_shape[h] is not None:
                res.append(tuple(layer.a_shape[h]))
            else:
                res.append((layer.n_vert[h], layer.n_slash[h]))
        return res

    kind_of = [c["kind"] for c in configs]
    start = sizes()
    hist = layer.refine_chunk(qc, c0, rows, out, lse=lse, threshold=0.9, max_rounds=3)
    torch.cuda.synchronize()
    cur = start
    for r in range(len(hist) - 1):
        nxt, raised = oracle.refine_sizes(hist[r], kind_of, cur, c1)
        assert raised.any()
        assert np.all(hist[r + 1][raised] >= hist[r][raised] - 1e-5)
        cur = nxt
    final, _ = oracle.refine_sizes(hist[-1], kind_of, cur, c1)
    assert sizes() == cur, (sizes(), cur)
    print(f"[refine] {len(hist) - 1} rounds; sizes {start} -> {cur}", flush=True)
    # final rows against the oracle on the final patterns
    verts, slashes = layer.pattern.lists()
    bidx, bcnt = layer.block_pattern.idx.cpu().numpy(), layer.block_pattern.cnt.cpu().numpy()
    qo, _, _ = oracle_inputs(q, k[:1], v[:1])
    ctxs = _contexts(cfg, k, v, c1)
    G = cfg.n_heads // cfg.n_kv_heads
    r = c0 + off
    for h in range(cfg.n_heads):
        if layer.blocks[h] is not None:
            kept = lambda i, h=h: bidx[h, (i - c0) // 64, :bcnt[h, (i - c0) // 64]]  # noqa
            ro, rl, _ = oracle.block_sparse_rows(qo[h, r], r, ctxs[h // G], kept, layer.sm_scale)
        else:
            if layer.a_shape[h] is not None:
                ov, os_ = oracle.a_shape_lists(*layer.a_shape[h], c1)
            else:
                ov, os_ = verts[h].numpy(), slashes[h].numpy()
            ro, rl, _ = oracle.sparse_rows(qo[h, r], r, ctxs[h // G], ov, os_, layer.sm_scale)
        compare(host64(out[h, off]), ro)
        lse_compare(host64(lse[h, off]), rl)
