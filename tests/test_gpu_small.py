"""GPU parity of every entry point on small inputs (HIP path through the C
ABI vs the fp64 oracle)."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import TINY, SEVEN_B_128K, scaled
from tests.gpu_util import (DEV, MAX_ABS, MEAN_ABS, compare, dca_of, host64, lse_compare,
                            near_tie_check, oracle_freqs, oracle_inputs, product_sm, rope_of,
                            score_compare)

pytestmark = pytest.mark.gpu

L = pytest.importorskip("long_context_sparse_rope_amd")


# ---------------------------------------------------------------- RoPE / DCA
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("blend", [False, True])
def test_rope_yarn_apply(dtype, blend, out_dtype):
    torch.manual_seed(0)
    H, n, D = 3, 300, 128
    x = torch.randn(H, n, D, device=DEV).to(dtype)
    pos = torch.randint(0, 1 << 20, (n,), dtype=torch.int32, device=DEV)
    pos[:4] = torch.tensor([0, 1, 262143, (1 << 30) - 1], dtype=torch.int32)
    rope = L.RopeConfig(base=1e7, yarn_factor=4.0, orig_max_pos=262144, freq_blend=blend)
    y = L.rope_yarn_apply(x, pos, rope, scale=1.25, out_dtype=out_dtype)
    assert y.dtype == out_dtype
    xs = oracle_inputs(x, x, x)[0]      # fp32 inputs are rounded to bf16 on entry
    th = (oracle.yarn_inv_freq(D, 1e7, 4.0, 262144) if blend else oracle.rope_inv_freq(D, 1e7))
    ref = oracle.rope_apply(xs, pos.cpu().numpy(), th, scale=1.25)
    got = host64(y)
    # the store: half an ulp (2^-9 relative for bf16, 2^-12 for fp16) plus
    # the fp32 rotation error
    half_ulp = 2.0 ** -9 if out_dtype == torch.bfloat16 else 2.0 ** -12
    assert np.all(np.abs(got - ref) <= 2 * half_ulp * np.abs(ref) + 1e-5)


def test_rope_no_rotate_and_inplace():
    x = torch.randn(2, 50, 64, device=DEV)
    y = L.rope_yarn_apply(x, None, L.RopeConfig(), rotate=False)
    assert torch.equal(y.float().cpu(), torch.from_numpy(oracle.bf16_round(x.cpu().numpy())))
    xb = torch.randn(2, 50, 64, device=DEV).to(torch.bfloat16)
    ref = host64(xb)
    pos = torch.arange(50, dtype=torch.int32, device=DEV)
    L.rope_yarn_apply(xb, pos, L.RopeConfig(base=1e4), out=xb)
    exp = oracle.rope_rotate(ref, np.arange(50), oracle.rope_inv_freq(64, 1e4))
    assert np.all(np.abs(host64(xb) - exp) <= 2.0 ** -8 * np.abs(exp) + 1e-5)


@pytest.mark.parametrize("chunk,local,start,n", [(0, 0, 0, 100), (256, 64, 0, 1024),
                                                 (262144, 32768, 1015808, 32768),
                                                 (8, 2, 5, 40)])
def test_dca_positions(chunk, local, start, n):
    out = L.dca_positions(start, n, L.DcaConfig(chunk, local), DEV)
    ref = oracle.dca_position_maps(np.arange(start, start + n), chunk, local)
    for k in ("pk", "intra", "succ", "inter"):
        assert out[k].cpu().numpy().astype(np.int64).tolist() == ref[k].tolist(), k


# ---------------------------------------------------------------- selection
@pytest.mark.parametrize("n,k", [(1000, 32), (4096, 1000), (50, 64), (100000, 6096), (37, 0),
                                 (3 * 16384 + 5, 4000), (1 << 20, 6096), (70000, 70000)])
def test_topk_select_only_bit_exact(n, k):
    rng = np.random.default_rng(n + k)
    H = 3
    v = rng.random((H, n)).astype(np.float32)
    v[:, ::7] = np.float32(0.5)                 # many exact ties
    v[0, 1::11] = -v[0, 1::11]                  # negative scores
    v[0, 2::13] = np.float32(-0.0)              # -0 ranks as +0
    v[1] = np.round(v[1] * 8) / 8               # coarse values: heavy ties
    s = rng.random((H, n)).astype(np.float32) ** 4
    s[2, :] = 0.0                               # all-equal head
    vs, ss = torch.from_numpy(v).to(DEV), torch.from_numpy(s).to(DEV)
    q = torch.zeros(H, 1, 64, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(1, n, 64, dtype=torch.float16, device=DEV)
    pat = L.Pattern(H, max(k, 1) + 5, max(k, 1) + 5, DEV)
    L.vs_pattern_estimate(q, kc, n - 1, L.RopeConfig(), L.DcaConfig(), 0.125, [k] * H, [k] * H,
                          pat, vert_score=vs, slash_score=ss, select_only=True)
    verts, slashes = pat.lists()
    for h in range(H):
        assert verts[h].tolist() == oracle.select_top(v[h], k).tolist()
        assert slashes[h].tolist() == oracle.select_top(s[h], k).tolist()
    vi = pat.vert_idx.cpu()
    assert torch.all(vi[:, min(k, n):] == -1)


# ---------------------------------------------------------------- estimate
def _tiny_layer(cfg, q, k, v, upto):
    layer = L.ChunkedSparsePrefill(cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len,
                                   rope_of(cfg), dca_of(cfg),
                                   product_sm(cfg),
                                   cfg.n_vert, cfg.n_slash, cfg.last_q, DEV)
    from tests.gpu_util import build_cache
    build_cache(layer, k, v, upto)
    return layer


@pytest.mark.parametrize("c0,lc", [(0, 1024), (768, 256), (0, 200), (512, 100)])
def test_estimate_scores_and_selection_tiny(c0, lc):
    cfg = TINY
    q, k, v = synth.generate(cfg, DEV)
    layer = _tiny_layer(cfg, q, k, v, c0 + lc)
    c1 = c0 + lc
    vs = torch.empty(1, c1, device=DEV)
    ss = torch.empty(1, c1, device=DEV)
    L.vs_pattern_estimate(q[:, c0:c1], layer.k_cache[:, :c1], c0, layer.rope, layer.dca,
                          layer.sm_scale, [32], [64], layer.pattern, vert_score=vs,
                          slash_score=ss)
    qo, ko, _ = oracle_inputs(q, k, v)
    ctx = oracle.KeyContext(ko[0, :c1], None, oracle_freqs(cfg), cfg.dca_chunk, cfg.dca_local)
    rows = oracle.estimate.estimate_rows(c0, lc, 64)
    rv, rs = oracle.estimate_scores(qo[0, rows], rows, ctx, c1, layer.sm_scale)
    gv, gs = host64(vs[0]), host64(ss[0])
    n_rows = len(rows)
    assert abs(gv.sum() - n_rows) < 1e-3 * n_rows and abs(gs.sum() - n_rows) < 1e-3 * n_rows
    score_compare(gv, rv, "vertical")
    score_compare(gs, rs, "slash")
    # selection from the GPU's own scores is the oracle's selection of them
    verts, slashes = layer.pattern.lists()
    assert verts[0].tolist() == oracle.select_top(vs[0].cpu().numpy(), 32).tolist()
    assert slashes[0].tolist() == oracle.select_top(ss[0].cpu().numpy(), 64).tolist()
    # and agrees with the fp64 selection except on near-ties
    near_tie_check(verts[0].numpy(), rv, 32, "vertical")
    near_tie_check(slashes[0].numpy(), rs, 64, "slash")


def test_estimate_deterministic():
    cfg = TINY
    q, k, v = synth.generate(cfg, DEV)
    layer = _tiny_layer(cfg, q, k, v, 1024)
    outs = []
    for _ in range(2):
        vs = torch.empty(1, 1024, device=DEV)
        ss = torch.empty(1, 1024, device=DEV)
        L.vs_pattern_estimate(q, layer.k_cache[:, :1024], 0, layer.rope, layer.dca,
                              layer.sm_scale, [32], [64], layer.pattern, vert_score=vs,
                              slash_score=ss)
        outs.append((vs.cpu(), ss.cpu(), layer.pattern.vert_idx.cpu().clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][2], outs[1][2])


# ---------------------------------------------------------------- attention
def _attn_case(cfg, c0, lc, verts, slashes, dense=False, out_dtype=torch.float32):
    q, k, v = synth.generate(cfg, DEV, n_tokens=c0 + lc)
    c1 = c0 + lc
    layer = _tiny_layer(cfg, q, k, v, c1)
    H = cfg.n_heads
    pat = None if dense else L.Pattern.from_lists(verts, slashes, DEV)
    out = torch.empty(H, lc, cfg.head_dim, dtype=out_dtype, device=DEV)
    lse = torch.empty(H, lc, device=DEV)
    stats = torch.zeros(2, dtype=torch.int64, device=DEV)
    L.vs_sparse_attn_prefill(q[:, c0:c1], layer.k_cache[:, :c1], layer.v_cache[:, :c1], c0,
                             layer.rope, layer.dca, layer.sm_scale, pat,
                             out=out, lse=lse, stats=stats, dense=dense)
    torch.cuda.synchronize()
    qo, ko, vo = oracle_inputs(q, k, v)
    th = oracle_freqs(cfg)
    G = cfg.group
    sizes_total = 0
    for h in range(H):
        ctx = oracle.KeyContext(ko[h // G, :c1], vo[h // G, :c1], th, cfg.dca_chunk,
                                cfg.dca_local)
        rows = np.arange(c0, c1)
        if dense:
            ro, rl = oracle.dense_causal_rows(qo[h, c0:c1], rows, ctx, layer.sm_scale)
            sizes = rows + 1
        else:
            ro, rl, sizes = oracle.sparse_rows(qo[h, c0:c1], rows, ctx, np.array(verts[h]),
                                               np.array(slashes[h]), layer.sm_scale)
        if out_dtype == torch.bfloat16:
            # the bf16 store adds up to half an ulp of |O| on top of the fp32 bar
            g = host64(out[h])
            d = np.abs(g - ro)
            assert np.all(d <= MAX_ABS + 2.0 ** -9 * np.abs(ro)), d.max()
            assert d.mean() <= MEAN_ABS + np.mean(2.0 ** -9 * np.abs(ro))
        else:
            compare(host64(out[h]), ro)
        lse_compare(host64(lse[h]), rl)
        sizes_total += int(np.sum(sizes))
    st = stats.cpu().tolist()
    assert st[1] == sizes_total, (st, sizes_total)
    assert st[0] >= st[1]
    return st


def test_attention_tiny_oracle_pattern():
    cfg = TINY
    q, k, v = synth.generate(cfg)
    qo, ko, _ = oracle_inputs(q, k, v)
    ctx = oracle.KeyContext(ko[0], None, oracle_freqs(cfg), cfg.dca_chunk, cfg.dca_local)
    rows = oracle.estimate.estimate_rows(0, 1024, 64)
    rv, rs = oracle.estimate_scores(qo[0, rows], rows, ctx, 1024, oracle.softmax_scale(64, 1.0))
    vsel, ssel = oracle.select_pattern(rv, rs, 32, 64)
    _attn_case(cfg, 0, 1024, [vsel.tolist()], [ssel.tolist()])


@pytest.mark.parametrize("c0,lc", [(0, 1024), (256, 300), (640, 384), (0, 77)])
def test_attention_tiny_random_pattern(c0, lc):
    rng = np.random.default_rng(c0 + lc)
    c1 = c0 + lc
    verts = [sorted(rng.choice(c1, size=min(40, c1), replace=False).tolist())]
    slashes = [sorted(set([0, 1, 2] + rng.choice(c1, size=min(60, c1), replace=False).tolist()))]
    _attn_case(TINY, c0, lc, verts, slashes)


@pytest.mark.parametrize("c0,lc", [(0, 1024), (192, 500)])
def test_attention_tiny_dense(c0, lc):
    _attn_case(TINY, c0, lc, None, None, dense=True)


# A DCA period that is a multiple of 32 but not of 64 (C 256, W 96: S 160):
# the walk cuts the key tiles [128, 192), [448, 512), ... at the chunk edges
# 160, 480, ..., and the row blocks on either side take different variants.
TINY_S160 = scaled(TINY, dca_local=96)
TINY_S208 = scaled(TINY, dca_local=48)


@pytest.mark.parametrize("c0,lc", [(0, 1024), (128, 448)])
def test_attention_period_160(c0, lc):
    rng = np.random.default_rng(160 + c0)
    c1 = c0 + lc
    verts = [sorted(rng.choice(c1, size=40, replace=False).tolist())]
    slashes = [sorted(set([0, 1, 2, 150, 159, 160, 161] +
                          rng.choice(c1, size=60, replace=False).tolist()))]
    _attn_case(TINY_S160, c0, lc, verts, slashes)
    _attn_case(TINY_S160, c0, lc, None, None, dense=True)


def test_estimate_period_208():
    """Estimate scores at S 208: 64-key tiles meet the chunk edges 208, 416,
    624 and 832, and each key takes its own chunk's rotation."""
    cfg = TINY_S208
    q, k, v = synth.generate(cfg, DEV)
    layer = _tiny_layer(cfg, q, k, v, 1024)
    vs = torch.empty(1, 1024, device=DEV)
    ss = torch.empty(1, 1024, device=DEV)
    L.vs_pattern_estimate(q[:, 0:1024], layer.k_cache[:, :1024], 0, layer.rope, layer.dca,
                          layer.sm_scale, [32], [64], layer.pattern, vert_score=vs,
                          slash_score=ss)
    qo, ko, _ = oracle_inputs(q, k, v)
    ctx = oracle.KeyContext(ko[0], None, oracle_freqs(cfg), cfg.dca_chunk, cfg.dca_local)
    rows = oracle.estimate.estimate_rows(0, 1024, 64)
    rv, rs = oracle.estimate_scores(qo[0, rows], rows, ctx, 1024, layer.sm_scale)
    score_compare(host64(vs[0]), rv, "vertical")
    score_compare(host64(ss[0]), rs, "slash")


def test_estimate_multi_tile_splits_with_dca_edges():
    """Estimate scores where every key split holds several tiles (the slash
    sums carried from tile to tile and added across split boundaries) and the
    DCA period (S 2800, four query heads, one per KV head) puts chunk edges
    inside tiles; every head, every score, and the selection."""
    cfg = scaled(TINY, n_heads=4, n_kv_heads=4, seq_len=40000, dca_chunk=3000,
                 dca_local=200, n_vert=96, n_slash=160)
    n = cfg.seq_len
    q, k, v = synth.generate(cfg, DEV)
    layer = _tiny_layer(cfg, q, k, v, n)
    c0 = 39040  # a multiple of 64, as DCA chunk starts must be
    vs = torch.empty(4, n, device=DEV)
    ss = torch.empty(4, n, device=DEV)
    L.vs_pattern_estimate(q[:, c0:n], layer.k_cache[:, :n], c0, layer.rope, layer.dca,
                          layer.sm_scale, [96] * 4, [160] * 4, layer.pattern, vert_score=vs,
                          slash_score=ss)
    qo, ko, _ = oracle_inputs(q, k, v)
    rows = oracle.estimate.estimate_rows(c0, n - c0, 64)
    verts, slashes = layer.pattern.lists()
    for h in range(4):
        ctx = oracle.KeyContext(ko[h], None, oracle_freqs(cfg), cfg.dca_chunk, cfg.dca_local)
        rv, rs = oracle.estimate_scores(qo[h, rows], rows, ctx, n, layer.sm_scale)
        score_compare(host64(vs[h]), rv, f"vertical h{h}")
        score_compare(host64(ss[h]), rs, f"slash h{h}")
        assert verts[h].tolist() == oracle.select_top(vs[h].cpu().numpy(), 96).tolist()
        assert slashes[h].tolist() == oracle.select_top(ss[h].cpu().numpy(), 160).tolist()
        near_tie_check(slashes[h].numpy(), rs, 160, f"slash h{h}")


def test_attention_empty_rows_and_bf16_out():
    # no slash 0 and verticals only far ahead: the first rows have empty sets
    _attn_case(TINY, 0, 256, [[200, 201]], [[150, 151]], out_dtype=torch.bfloat16)


def test_attention_gqa_d128_dca():
    cfg = scaled(SEVEN_B_128K, n_heads=4, n_kv_heads=2, seq_len=2048, dca_chunk=1024,
                 dca_local=256, n_vert=64, n_slash=128)
    rng = np.random.default_rng(7)
    verts, slashes = [], []
    for h in range(4):
        verts.append(sorted(set(rng.choice(2048, 64, replace=False).tolist())))
        slashes.append(sorted(set(list(range(0, 100)) +
                                  rng.choice(2048, 28, replace=False).tolist())))
    _attn_case(cfg, 1024, 1024, verts, slashes)
    _attn_case(cfg, 640, 384, verts, slashes)


# ---------------------------------------------------------------- recall
def test_recall_tiny():
    cfg = TINY
    q, k, v = synth.generate(cfg, DEV)
    layer = _tiny_layer(cfg, q, k, v, 1024)
    layer.estimate(q, 0)
    rows = torch.tensor([0, 5, 100, 223, 224, 500, 959, 1023], dtype=torch.int32, device=DEV)
    lf, ls, rc = layer.recall(q, 0, rows)
    verts, slashes = layer.pattern.lists()
    qo, ko, vo = oracle_inputs(q, k, v)
    ctx = oracle.KeyContext(ko[0], vo[0], oracle_freqs(cfg), cfg.dca_chunk, cfg.dca_local)
    r = rows.cpu().numpy().astype(np.int64)
    of, os_, orc = oracle.attention_recall(qo[0, r], r, ctx, verts[0].numpy(), slashes[0].numpy(),
                                           layer.sm_scale)
    lse_compare(host64(lf[0]), of)
    lse_compare(host64(ls[0]), os_)
    assert np.max(np.abs(host64(rc[0]) - orc)) < 1e-2
