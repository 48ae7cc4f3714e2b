"""GPU parity of the decode-step attention (lcsr_attn_decode) through the C
ABI against the fp64 oracle's dense causal rows, with the same DCA logits:
single rows and short row runs, rows beside DCA period and local-window
edges, the 32-matrix-row maximum, grouped heads at D 128, bf16 output, and
bitwise reproducibility."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import TINY, SEVEN_B_128K, scaled
from tests.gpu_util import (DEV, MAX_ABS, MEAN_ABS, build_cache, compare, dca_of, host64,
                            lse_compare, oracle_freqs, oracle_inputs, product_sm, rope_of)

pytestmark = pytest.mark.gpu

L = pytest.importorskip("long_context_sparse_rope_amd")


def _layer(cfg, k, v):
    layer = L.ChunkedSparsePrefill(cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len,
                                   rope_of(cfg), dca_of(cfg),
                                   product_sm(cfg),
                                   cfg.n_vert, cfg.n_slash, cfg.last_q, DEV)
    build_cache(layer, k, v, cfg.seq_len)
    return layer


def _decode_case(cfg, q, k, v, layer, p0, n, out_dtype=torch.float32):
    """Rows p0 .. p0 + n - 1 against every key up to each row."""
    c1 = p0 + n
    print(f"[decode] {cfg.name} rows {p0}..{c1 - 1}", flush=True)
    H = cfg.n_heads
    lse = torch.empty(H, n, device=DEV)
    out, _ = L.attn_decode(q[:, p0:c1], layer.k_cache[:, :c1], layer.v_cache[:, :c1], p0,
                           layer.rope, layer.dca, layer.sm_scale, out_dtype=out_dtype, lse=lse)
    torch.cuda.synchronize()
    qo, ko, vo = oracle_inputs(q, k, v)
    th = oracle_freqs(cfg)
    G = cfg.group
    rows = np.arange(p0, c1)
    for h in range(H):
        ctx = oracle.KeyContext(ko[h // G, :c1], vo[h // G, :c1], th, cfg.dca_chunk,
                                cfg.dca_local)
        ro, rl = oracle.dense_causal_rows(qo[h, p0:c1], rows, ctx, layer.sm_scale)
        if out_dtype == torch.bfloat16:
            d = np.abs(host64(out[h]) - ro)
            assert np.all(d <= MAX_ABS + 2.0 ** -9 * np.abs(ro)), d.max()
            assert d.mean() <= MEAN_ABS + np.mean(2.0 ** -9 * np.abs(ro))
        else:
            compare(host64(out[h]), ro)
        lse_compare(host64(lse[h]), rl)
    return out, lse


@pytest.fixture(scope="module")
def tiny():
    cfg = TINY
    assert cfg.dca_chunk - cfg.dca_local == 224
    q, k, v = synth.generate(cfg, DEV)
    return cfg, q, k, v, _layer(cfg, k, v)


# TINY: one head, D 64, DCA C 256, W 32 (period S 224), 1024 tokens.  The
# rows (222, 4), (447, 3), (670, 4) and (894, 3) straddle the period edges 224,
# 448, 672 and 896: their earlier rows meet keys of the next DCA chunk, all
# masked for them.  The 64-key tiles 192..255 and 640..703 hold an edge:
# their keys on either side take their own chunk's query variant.
@pytest.mark.parametrize("p0,n", [(1023, 1), (0, 1), (1, 3), (1000, 24), (222, 4),
                                  (447, 3), (670, 4), (894, 3), (255, 2), (190, 4),
                                  (480, 32), (63, 2), (700, 17)])
def test_decode_tiny(tiny, p0, n):
    cfg, q, k, v, layer = tiny
    _decode_case(cfg, q, k, v, layer, p0, n)


def test_decode_period_208():
    """DCA period S 208 (C 256, W 48), a multiple of 16 only: the 64-key tiles
    192..255 and 384..447 hold the chunk edges 208 and 416; rows on both sides
    of each edge."""
    cfg = scaled(TINY, dca_local=48)
    q, k, v = synth.generate(cfg, DEV)
    layer = _layer(cfg, k, v)
    for p0, n in ((206, 4), (414, 3), (255, 2), (1023, 1), (600, 16)):
        _decode_case(cfg, q, k, v, layer, p0, n)


def test_decode_tiny_bf16_out_and_reproducible(tiny):
    cfg, q, k, v, layer = tiny
    o1, l1 = _decode_case(cfg, q, k, v, layer, 900, 8, out_dtype=torch.bfloat16)
    o2, l2 = _decode_case(cfg, q, k, v, layer, 900, 8, out_dtype=torch.bfloat16)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_gqa_d128_dca():
    """Seven query heads per KV head (the 7B grouping) at D 128 with DCA:
    up to 4 rows fill 28 of the 32 matrix rows; rows beside the period edge
    (S = 768) and the local window (S + 256)."""
    cfg = scaled(SEVEN_B_128K, n_heads=14, n_kv_heads=2, seq_len=4096, dca_chunk=1024,
                 dca_local=256, n_vert=64, n_slash=128)
    q, k, v = synth.generate(cfg, DEV)
    layer = _layer(cfg, k, v)
    for p0, n in ((4095, 1), (3000, 4), (766, 4), (1022, 3), (64, 1)):
        _decode_case(cfg, q, k, v, layer, p0, n)


def test_decode_matches_dense_prefill_rows(tiny):
    """The decode rows equal the dense prefill's rows of the same chunk (two
    work splits of one definition), to rounding."""
    cfg, q, k, v, layer = tiny
    c0, lc = 960, 32
    out_p = torch.empty(1, lc, cfg.head_dim, device=DEV)
    L.vs_sparse_attn_prefill(q[:, c0:c0 + lc], layer.k_cache[:, :c0 + lc],
                             layer.v_cache[:, :c0 + lc], c0, layer.rope, layer.dca,
                             layer.sm_scale, None, out=out_p, dense=True)
    out_d, _ = L.attn_decode(q[:, c0:c0 + lc], layer.k_cache[:, :c0 + lc],
                             layer.v_cache[:, :c0 + lc], c0, layer.rope, layer.dca,
                             layer.sm_scale)
    d = (out_p - out_d).abs().max().item()
    assert d <= 1e-3, d


def test_decode_graph_replay(tiny):
    """The decode call with caller-owned output, lse and workspace launches
    kernels only, so it can be captured in a HIP graph: every replay (with
    eager work and synchronisations between them, and new query values
    copied into the captured input) equals the eager call."""
    cfg, q, k, v, layer = tiny
    p0, n = 1000, 8
    qs = q[:, p0:p0 + n].clone()
    args = (layer.k_cache[:, :p0 + n], layer.v_cache[:, :p0 + n], p0, layer.rope, layer.dca,
            layer.sm_scale)
    ws = torch.empty(L.workspace_bytes(L._capi.LCSR_WS_DECODE, qs, args[0], p0, layer.rope,
                                       layer.dca), dtype=torch.uint8, device=DEV)
    out = torch.empty(cfg.n_heads, n, cfg.head_dim, device=DEV)
    lse = torch.empty(cfg.n_heads, n, device=DEV)
    L.attn_decode(qs, *args, out=out, lse=lse, workspace=ws)   # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.attn_decode(qs, *args, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        src = q[:, p0 - 100 * rep:p0 - 100 * rep + n]
        qs.copy_(src)
        ref_o, _ = L.attn_decode(src.contiguous(), *args, lse=(ref_l := torch.empty_like(lse)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), rep
