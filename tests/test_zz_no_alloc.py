"""lcsr_attn_decode_noalloc, the decode step on the library's static scratch,
against lcsr_attn_decode with a caller-owned workspace: two calls in a row,
the second on a smaller problem (fewer rows, a shorter cache, fewer key
splits), each bitwise equal to the workspace call and within the fp64
oracle's bar."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import SEVEN_B_128K, scaled
from tests.gpu_util import (DEV, build_cache, compare, dca_of, lse_compare, oracle_freqs,
                            oracle_inputs, product_sm, rope_of)

pytestmark = pytest.mark.gpu

L = pytest.importorskip("long_context_sparse_rope_amd")

# the 7B grouping at D 128 with DCA (period S = 768)
CFG = scaled(SEVEN_B_128K, n_heads=14, n_kv_heads=2, seq_len=4096, dca_chunk=1024,
             dca_local=256, n_vert=64, n_slash=128)


def test_decode_noalloc_matches_workspace_call():
    cfg = CFG
    q, k, v = synth.generate(cfg, DEV)
    layer = L.ChunkedSparsePrefill(cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len,
                                   rope_of(cfg), dca_of(cfg), product_sm(cfg), cfg.n_vert,
                                   cfg.n_slash, cfg.last_q, DEV)
    build_cache(layer, k, v, cfg.seq_len)
    qo, ko, vo = oracle_inputs(q, k, v)
    th = oracle_freqs(cfg)
    sm = oracle.softmax_scale(cfg.head_dim, cfg.yarn_factor)
    H = cfg.n_heads
    for p0, n in ((4092, 4), (766, 2)):
        c1 = p0 + n
        print(f"[noalloc] rows {p0}..{c1 - 1}", flush=True)
        args = (layer.k_cache[:, :c1], layer.v_cache[:, :c1], p0, layer.rope, layer.dca,
                layer.sm_scale)
        ref_l = torch.empty(H, n, device=DEV)
        ref, _ = L.attn_decode(q[:, p0:c1], *args, lse=ref_l)
        out = torch.full_like(ref, float("nan"))
        lse = torch.full_like(ref_l, float("nan"))
        L.attn_decode_noalloc(q[:, p0:c1], *args, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, ref_l), (p0, n)
        rows = np.arange(p0, c1)
        for g in range(cfg.n_kv_heads):
            h = g * cfg.group + (p0 % cfg.group)
            ctx = oracle.KeyContext(ko[g, :c1], vo[g, :c1], th, cfg.dca_chunk, cfg.dca_local)
            ro, rl = oracle.dense_causal_rows(qo[h, p0:c1], rows, ctx, sm)
            compare(out[h].cpu().numpy().astype(np.float64), ro)
            lse_compare(lse[h].cpu().numpy().astype(np.float64), rl)
