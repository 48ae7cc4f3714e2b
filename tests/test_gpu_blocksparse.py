"""GPU parity of the block-sparse pattern through the C ABI against the fp64
oracle: block scores, the selection (bit-exact on identical scores, ties and
signed zeros included), attention over the kept blocks on every row with
exact pair counts, every block kept = the dense kernel, and a ragged chunk
of the fp32 tiny layer."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import FOURTEEN_B_256K, SEVEN_B_128K, TINY, scaled
from tests.gpu_util import (DEV, build_cache, compare, dca_of, host64, lse_compare,
                            oracle_freqs, oracle_inputs, product_sm, rope_of)

pytestmark = pytest.mark.gpu

L = pytest.importorskip("long_context_sparse_rope_amd")

# 7B grouping at D 128 with DCA (period S = 768); the chunk [3072, 4096)
# sees keys in DCA chunks 0 .. 5
CFG = scaled(SEVEN_B_128K, n_heads=14, n_kv_heads=2, seq_len=4096, prefill_chunk=1024,
             dca_chunk=1024, dca_local=256, n_vert=64, n_slash=128)


# the 14B grouping (5 query heads per KV head) at the same small shape
CFG14 = scaled(FOURTEEN_B_256K, n_heads=10, n_kv_heads=2, seq_len=4096, prefill_chunk=1024,
               dca_chunk=1024, dca_local=256, n_vert=64, n_slash=128)


def _layer(cfg):
    return L.ChunkedSparsePrefill(cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len,
                                  rope_of(cfg), dca_of(cfg),
                                  product_sm(cfg),
                                  cfg.n_vert, cfg.n_slash, cfg.last_q, DEV)


def _contexts(cfg, k, v, upto):
    _, ko, vo = oracle_inputs(k[:1], k, v)
    th = oracle_freqs(cfg)
    return [oracle.KeyContext(ko[g, :upto], vo[g, :upto], th, cfg.dca_chunk, cfg.dca_local) for g in range(cfg.n_kv_heads)]


def _estimate(layer, q, c0, c1, budgets, max_blocks):
    H = q.shape[0]
    n_qb, n_kb = -(-(c1 - c0) // 64), -(-c1 // 64)
    pat = L.BlockPattern(H, n_qb, max_blocks, DEV)
    sc = torch.full((H, n_qb, n_kb), float("nan"), device=DEV)
    L.block_sparse_estimate(q[:, c0:c1], layer.k_cache[:, :c1], c0, layer.rope, layer.dca,
                            layer.sm_scale, budgets, pat, scores=sc)
    torch.cuda.synchronize()
    return pat, sc


def _check_selection(pat, scores, c0, budgets):
    """The oracle's rule on the GPU's own fp32 scores, every (head, block)."""
    idx, cnt = pat.idx.cpu().numpy(), pat.cnt.cpu().numpy()
    sc = scores.cpu().numpy().astype(np.float64)
    H, n_qb = cnt.shape
    for h in range(H):
        for qb in range(n_qb):
            diag = c0 // 64 + qb
            ref = oracle.select_blocks(sc[h, qb, :diag + 1], diag, budgets[h])
            assert cnt[h, qb] == ref.size, (h, qb)
            np.testing.assert_array_equal(idx[h, qb, :ref.size], ref)
            assert np.all(idx[h, qb, ref.size:] == -1)


def test_block_scores_and_selection():
    cfg = CFG
    q, k, v = synth.generate(cfg, DEV)
    layer = _layer(cfg)
    build_cache(layer, k, v, cfg.seq_len)
    c0, c1 = 3072, 4096
    budgets = [1, 2, 5, 8, 16, 64, 100] * 2
    pat, sc = _estimate(layer, q, c0, c1, budgets, 100)
    qo, _, _ = oracle_inputs(q, k[:1], v[:1])
    ctxs = _contexts(cfg, k, v, c1)
    G = cfg.n_heads // cfg.n_kv_heads
    got = host64(sc)
    worst = 0.0
    for h in range(cfg.n_heads):
        ref = oracle.block_scores(qo[h, c0:c1], c0, ctxs[h // G], layer.sm_scale)
        fin = np.isfinite(ref)
        d = np.abs(got[h][fin] - ref[fin])
        worst = max(worst, float(np.max(d / (1e-3 + np.abs(ref[fin])))))
        assert np.all(d <= 1e-4 + 1e-4 * np.abs(ref[fin])), (h, d.max())
    print(f"[block] score worst relative error {worst:.2e}", flush=True)
    _check_selection(pat, sc, c0, budgets)
    # select-only on the same scores gives the same lists
    pat2 = L.BlockPattern(cfg.n_heads, pat.idx.shape[1], 100, DEV)
    L.block_sparse_estimate(q[:, c0:c1], layer.k_cache[:, :c1], c0, layer.rope, layer.dca,
                            layer.sm_scale, budgets, pat2, scores=sc, select_only=True)
    torch.cuda.synchronize()
    assert torch.equal(pat.idx, pat2.idx) and torch.equal(pat.cnt, pat2.cnt)


def test_selection_ties_and_signed_zeros():
    """Constructed scores: few distinct values (many ties), +0 and -0."""
    H, c0, c1 = 3, 2048, 2048 + 640
    n_qb, n_kb = 10, -(-c1 // 64)
    rng = np.random.default_rng(5)
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 3.0], dtype=np.float32)
    sc_h = vals[rng.integers(0, vals.size, size=(H, n_qb, n_kb))]
    sc = torch.from_numpy(sc_h).to(DEV)
    q = torch.zeros(H, c1 - c0, 64, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(1, c1, 64, dtype=torch.float16, device=DEV)
    budgets = [3, 17, 41]
    pat = L.BlockPattern(H, n_qb, 64, DEV)
    L.block_sparse_estimate(q, kc, c0, L.RopeConfig(base=1e4), L.DcaConfig(0, 0), 0.125,
                            budgets, pat, scores=sc, select_only=True)
    torch.cuda.synchronize()
    _check_selection(pat, sc, c0, budgets)


@pytest.mark.parametrize("cfg", [CFG, CFG14], ids=["group7", "group5"])
def test_block_sparse_attention_rows(cfg):
    q, k, v = synth.generate(cfg, DEV)
    layer = _layer(cfg)
    build_cache(layer, k, v, cfg.seq_len)
    c0, c1 = 3072, 4096
    budgets = ([4, 8, 1, 12, 6, 3, 20] * 2)[:cfg.n_heads]
    pat, _ = _estimate(layer, q, c0, c1, budgets, 20)
    H, n, D = cfg.n_heads, c1 - c0, cfg.head_dim
    out = torch.empty(H, n, D, device=DEV)
    lse = torch.empty(H, n, device=DEV)
    stats = torch.zeros(2, dtype=torch.int64, device=DEV)
    L.block_sparse_attn_prefill(q[:, c0:c1], layer.k_cache[:, :c1], layer.v_cache[:, :c1], c0,
                                layer.rope, layer.dca, layer.sm_scale, pat, out=out, lse=lse,
                                stats=stats)
    torch.cuda.synchronize()
    idx, cnt = pat.idx.cpu().numpy(), pat.cnt.cpu().numpy()
    qo, _, _ = oracle_inputs(q, k[:1], v[:1])
    ctxs = _contexts(cfg, k, v, c1)
    G = H // cfg.n_kv_heads
    rows = np.arange(c0, c1)
    pairs = 0
    for h in range(H):
        kept = lambda i, h=h: idx[h, (i - c0) // 64, :cnt[h, (i - c0) // 64]]  # noqa: E731
        ro, rl, sizes = oracle.block_sparse_rows(qo[h, rows], rows, ctxs[h // G], kept,
                                                 layer.sm_scale)
        print(f"[block] head {h} budget {budgets[h]}", flush=True)
        compare(host64(out[h]), ro)
        lse_compare(host64(lse[h]), rl)
        pairs += int(sizes.sum())
    assert int(stats[1].item()) == pairs


def test_shared_tiles_equal_per_head_kernel():
    """Lists that fit the shared-tile kernel (G x max_blocks <= 2048) and the
    same lists in wider buffers (per-head kernel) give bitwise the same rows:
    each head multiplies its own blocks in the same ascending order."""
    cfg = CFG
    q, k, v = synth.generate(cfg, DEV)
    layer = _layer(cfg)
    build_cache(layer, k, v, cfg.seq_len)
    c0, c1 = 3072, 4096
    budgets = [4, 8, 1, 12, 6, 3, 20] * 2
    pat, _ = _estimate(layer, q, c0, c1, budgets, 20)
    wide = L.BlockPattern(cfg.n_heads, pat.idx.shape[1], 300, DEV)
    wide.idx[:, :, :20] = pat.idx
    wide.cnt.copy_(pat.cnt)
    outs = []
    for pt in (pat, wide):
        o, lse = L.block_sparse_attn_prefill(
            q[:, c0:c1], layer.k_cache[:, :c1], layer.v_cache[:, :c1], c0, layer.rope,
            layer.dca, layer.sm_scale, pt, lse=torch.empty(cfg.n_heads, c1 - c0, device=DEV))
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_block_recall_rows():
    """lcsr_block_sparse_recall_check against the oracle: lse over the kept
    blocks, lse over every causal key, recall = exp of the difference."""
    cfg = CFG
    q, k, v = synth.generate(cfg, DEV)
    layer = _layer(cfg)
    build_cache(layer, k, v, cfg.seq_len)
    c0, c1 = 3072, 4096
    budgets = [2, 6, 16] * 4 + [1, 30]
    pat, _ = _estimate(layer, q, c0, c1, budgets, 30)
    off = np.array([0, 1, 63, 64, 500, 767, 768, 900, 1023])
    rows = torch.tensor(off, dtype=torch.int32, device=DEV)
    lf, ls, rc = L.block_sparse_recall_check(q[:, c0:c1], layer.k_cache[:, :c1], c0, layer.rope,
                                             layer.dca, layer.sm_scale, pat, rows)
    torch.cuda.synchronize()
    idx, cnt = pat.idx.cpu().numpy(), pat.cnt.cpu().numpy()
    qo, _, _ = oracle_inputs(q, k[:1], v[:1])
    ctxs = _contexts(cfg, k, v, c1)
    G = cfg.n_heads // cfg.n_kv_heads
    r = c0 + off
    for h in range(cfg.n_heads):
        kept = lambda i, h=h: idx[h, (i - c0) // 64, :cnt[h, (i - c0) // 64]]  # noqa: E731
        _, sl, _ = oracle.block_sparse_rows(qo[h, r], r, ctxs[h // G], kept, layer.sm_scale)
        _, fl = oracle.dense_causal_rows(qo[h, r], r, ctxs[h // G], layer.sm_scale)
        lse_compare(host64(lf[h]), fl)
        lse_compare(host64(ls[h]), sl)
        assert np.max(np.abs(host64(rc[h]) - np.exp(sl - fl))) < 1e-2, h


def test_every_block_is_dense():
    """A budget above the number of key blocks keeps every block: the rows
    equal the dense kernel's (two work splits of one definition)."""
    cfg = CFG
    q, k, v = synth.generate(cfg, DEV)
    layer = _layer(cfg)
    build_cache(layer, k, v, cfg.seq_len)
    c0, c1 = 2048, 3072
    nb = c1 // 64
    pat, _ = _estimate(layer, q, c0, c1, [nb] * cfg.n_heads, nb)
    assert torch.all(pat.cnt == (torch.arange(16, device=DEV) + c0 // 64 + 1)[None])
    ob, _ = L.block_sparse_attn_prefill(q[:, c0:c1], layer.k_cache[:, :c1],
                                        layer.v_cache[:, :c1], c0, layer.rope, layer.dca,
                                        layer.sm_scale, pat)
    od = torch.empty_like(ob)
    L.vs_sparse_attn_prefill(q[:, c0:c1], layer.k_cache[:, :c1], layer.v_cache[:, :c1], c0,
                             layer.rope, layer.dca, layer.sm_scale, None, out=od, dense=True)
    torch.cuda.synchronize()
    d = (ob - od).abs().max().item()
    assert d <= 1e-3, d


@pytest.mark.parametrize("local", [32, 48])
def test_tiny_ragged_chunk_bf16_out(local):
    """fp32 inputs (taken at bf16), D 64, DCA C 256 with W 32 (S 224) and W 48
    (S 208): key blocks 192..255 (and more) hold a chunk edge, query blocks
    too; a 1000-row chunk after 0 (last query block of 40 rows) and bf16
    output."""
    cfg = scaled(TINY, dca_local=local)
    q, k, v = synth.generate(cfg, DEV)
    layer = _layer(cfg)
    build_cache(layer, k, v, cfg.seq_len)
    c0, c1 = 0, 1000
    budgets = [5]
    pat, sc = _estimate(layer, q, c0, c1, budgets, 8)
    _check_selection(pat, sc, c0, budgets)
    qo, ko, vo = oracle_inputs(q, k, v)
    ctx = oracle.KeyContext(ko[0, :c1], vo[0, :c1], oracle_freqs(cfg), cfg.dca_chunk,
                            cfg.dca_local)
    ref_sc = oracle.block_scores(qo[0, c0:c1], c0, ctx, layer.sm_scale)
    fin = np.isfinite(ref_sc)
    assert np.all(np.abs(host64(sc[0])[fin] - ref_sc[fin]) <= 1e-4 + 1e-4 * np.abs(ref_sc[fin]))
    out, _ = L.block_sparse_attn_prefill(q[:, c0:c1], layer.k_cache[:, :c1],
                                         layer.v_cache[:, :c1], c0, layer.rope, layer.dca,
                                         layer.sm_scale, pat, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    idx, cnt = pat.idx.cpu().numpy(), pat.cnt.cpu().numpy()
    rows = np.arange(c0, c1)
    ro, _, _ = oracle.block_sparse_rows(qo[0, rows], rows, ctx,
                                        lambda i: idx[0, i // 64, :cnt[0, i // 64]],
                                        layer.sm_scale)
    d = np.abs(host64(out[0]) - ro)
    assert np.all(d <= 1e-2 + 2.0 ** -9 * np.abs(ro)), d.max()


def test_empty_chunk_is_a_no_op():
    """chunk_len 0: the block estimate, attention and recall succeed and write
    nothing; a decode call with no rows too."""
    cfg = CFG
    q, k, v = synth.generate(cfg, DEV)
    layer = _layer(cfg)
    build_cache(layer, k, v, 1024)
    H = cfg.n_heads
    pat = L.BlockPattern(H, 1, 4, DEV)
    pat.idx.fill_(7)
    pat.cnt.fill_(3)
    q0 = q[:, 1024:1024]
    L.block_sparse_estimate(q0, layer.k_cache[:, :1024], 1024, layer.rope, layer.dca,
                            layer.sm_scale, [4] * H, pat)
    out = torch.full((H, 0, cfg.head_dim), 5.0, device=DEV)
    L.block_sparse_attn_prefill(q0, layer.k_cache[:, :1024], layer.v_cache[:, :1024], 1024,
                                layer.rope, layer.dca, layer.sm_scale, pat, out=out)
    rows = torch.zeros(0, dtype=torch.int32, device=DEV)
    lf, _, _ = L.block_sparse_recall_check(q0, layer.k_cache[:, :1024], 1024, layer.rope,
                                           layer.dca, layer.sm_scale, pat, rows)
    od, _ = L.attn_decode(q0, layer.k_cache[:, :1024], layer.v_cache[:, :1024], 1024,
                          layer.rope, layer.dca, layer.sm_scale)
    torch.cuda.synchronize()
    assert torch.all(pat.idx == 7) and torch.all(pat.cnt == 3)
    assert lf.numel() == 0 and od.numel() == 0
