"""Parity at the full layer shapes, on sampled outputs.

Each layer (7B-shaped 128K, 14B-shaped 256K, 7B-shaped 1M with DCA and
YaRN s = 4, 14B-shaped 512K refinement stress) runs its whole chunk loop on
the GPU through the C ABI, in the launch configuration the benchmark times,
with the logit scale the library forms (lcsr_softmax_scale).  For a few
chunks per layer (the first, the ones that straddle a DCA key period or the
local window, the last) the run keeps:

* the estimate scores of every head, so that the selection can be checked
  bit for bit against the oracle's selection of the same fp32 scores;
* the attention output and lse of sampled rows: the chunk's estimate rows,
  its first rows, rows beside each DCA period edge (S k +- 2) and beside the
  local-window edge (S k + W - 1, S k + W), and 128 seeded rows.

The fp64 oracle (exact rotated operands) recomputes every query head on the
sampled rows of the last checked chunk and one head of every KV group on the
other checked chunks (a different head of the group per chunk), with the
GPU's own pattern; and the estimate scores of one head per KV group on the
last checked chunk, where the fp64 selection may differ from the GPU's only
on near-ties.  Every chunk's full output is checked to be finite.
"""

import functools

import numpy as np
import pytest
import torch

import long_context_sparse_rope_amd as L
import oracle
import synth
from synth.configs import CONFIGS, scaled
from tests.gpu_util import (DEV, MAX_ABS, MEAN_ABS, SCORE_REL, SCORE_REL_LARGE_LOGITS, compare,
                            critical_pair_total, dca_of, lse_compare, near_tie_check,
                            oracle_freqs, parallel_map, product_sm, rope_of, score_compare)

pytestmark = pytest.mark.gpu

CHECK_CHUNKS = {
    "7b_128k": (0, 3),
    "14b_256k": (0, 7),
    "7b_1m_dca": (7, 8, 31),
    "14b_512k_refine": (7, 8, 15),
    "14b_512k_unit_noise": (8, 15),
}
N_SEEDED_ROWS = 128
RECALL_ROWS = 16   # rows per oracle head in the recall check
DENSE_ROWS = 128   # dense-mode rows at the 1M context, spread over the KV groups


def group_heads(cfg, c):
    """One query head per KV group, a different one of the group per chunk."""
    return [g * cfg.group + (g + c) % cfg.group for g in range(cfg.n_kv_heads)]


def heads_of_chunk(cfg, c, last):
    return list(range(cfg.n_heads)) if c == last else group_heads(cfg, c)


def sample_rows(cfg, c0, lc):
    """Absolute rows of chunk [c0, c0 + lc) whose outputs are checked."""
    c1 = c0 + lc
    rows = set(range(max(c0, c1 - cfg.last_q), c1)) | set(range(c0, min(c1, c0 + 64)))
    if cfg.dca_chunk:
        S = cfg.dca_chunk - cfg.dca_local
        for kk in range(0, c1 // S + 1):
            for i in (S * kk - 2, S * kk - 1, S * kk, S * kk + 1, S * kk + 2,
                      S * kk + cfg.dca_local - 1, S * kk + cfg.dca_local):
                if c0 <= i < c1:
                    rows.add(i)
    rng = np.random.default_rng([cfg.seed, 7, c0])
    rows |= set(rng.choice(np.arange(c0, c1), size=min(N_SEEDED_ROWS, lc),
                           replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def _dca_twin(cfg, layer, q, k, v, res):
    """The 256K layer again with DCA on (C = 262,144 = the sequence, W =
    32,768): every causal relative position is then the plain one, so the
    estimate scores and, on the DCA-off pattern, the attention rows must
    agree with the DCA-off run to rounding."""
    C, W = 262144, 32768
    tw = scaled(cfg, dca_chunk=C, dca_local=W)
    sm = product_sm(tw)
    twin = L.ChunkedSparsePrefill(tw.n_heads, tw.n_kv_heads, tw.head_dim, tw.seq_len,
                                  rope_of(tw), dca_of(tw), sm, tw.n_vert, tw.n_slash,
                                  tw.last_q, DEV)
    out = torch.empty(tw.n_heads, tw.prefill_chunk, tw.head_dim, dtype=torch.float32, device=DEV)
    lse = torch.empty(tw.n_heads, tw.prefill_chunk, dtype=torch.float32, device=DEV)
    res["twin"] = {}
    for c in range(tw.n_chunks):
        c0, lc = tw.chunk_bounds(c)
        c1 = c0 + lc
        twin.append_kv(k[:, c0:c1], v[:, c0:c1], c0)
        if c not in CHECK_CHUNKS[cfg.name]:
            continue
        ch = res["chunks"][c]
        vs = torch.empty(tw.n_heads, c1, device=DEV)
        ss = torch.empty(tw.n_heads, c1, device=DEV)
        L.vs_pattern_estimate(q[:, c0:c1], twin.k_cache[:, :c1], c0, twin.rope, twin.dca, sm,
                              twin.n_vert, twin.n_slash, twin.pattern, last_q=tw.last_q,
                              vert_score=vs, slash_score=ss)
        pat = L.Pattern.from_lists(ch["verts"], ch["slashes"], DEV, max_vert=tw.n_vert,
                                   max_slash=tw.n_slash)
        L.vs_sparse_attn_prefill(q[:, c0:c1], twin.k_cache[:, :c1], twin.v_cache[:, :c1], c0,
                                 twin.rope, twin.dca, sm, pat, out=out[:, :lc], lse=lse[:, :lc])
        ri = torch.as_tensor(ch["rows"] - c0, device=DEV)
        res["twin"][c] = {"vs": vs.cpu().numpy(), "ss": ss.cpu().numpy(),
                          "out": out[:, ri].cpu().numpy(), "lse": lse[:, ri].cpu().numpy()}
    del twin


@functools.lru_cache(maxsize=1)
def run_layer(name):
    """Run the layer's chunk loop on the GPU; keep what the checks need."""
    cfg = CONFIGS[name]
    key_context.cache_clear()
    torch.cuda.empty_cache()
    q, k, v = synth.generate(cfg, DEV)
    sm = product_sm(cfg)
    H, D = cfg.n_heads, cfg.head_dim
    layer = L.ChunkedSparsePrefill(H, cfg.n_kv_heads, D, cfg.seq_len, rope_of(cfg),
                                   dca_of(cfg), sm, cfg.n_vert, cfg.n_slash, cfg.last_q, DEV)
    res = {"chunks": {}, "sm": oracle.softmax_scale(cfg.head_dim, cfg.yarn_factor)}
    out = torch.empty(H, cfg.prefill_chunk, D, dtype=torch.float32, device=DEV)
    lse = torch.empty(H, cfg.prefill_chunk, dtype=torch.float32, device=DEV)
    for c in range(cfg.n_chunks):
        c0, lc = cfg.chunk_bounds(c)
        c1 = c0 + lc
        qc = q[:, c0:c1]
        layer.append_kv(k[:, c0:c1], v[:, c0:c1], c0)
        keep = c in CHECK_CHUNKS[name]
        vs = ss = None
        if keep:
            vs = torch.empty(H, c1, device=DEV)
            ss = torch.empty(H, c1, device=DEV)
        L.vs_pattern_estimate(qc, layer.k_cache[:, :c1], c0, layer.rope, layer.dca, sm,
                              layer.n_vert, layer.n_slash, layer.pattern, last_q=cfg.last_q,
                              vert_score=vs, slash_score=ss)
        stats = torch.zeros(2, dtype=torch.int64, device=DEV)
        layer.attend(qc, c0, out=out[:, :lc], lse=lse[:, :lc], stats=stats)
        assert bool(torch.isfinite(out[:, :lc]).all()), f"non-finite output in chunk {c}"
        if keep:
            rows = sample_rows(cfg, c0, lc)
            ri = torch.as_tensor(rows - c0, device=DEV)
            verts, slashes = layer.pattern.lists()
            res["chunks"][c] = {
                "c0": c0, "lc": lc, "rows": rows,
                "q": q[:, torch.as_tensor(rows, device=DEV)].float().cpu().numpy(),
                "q_est": q[:, max(c0, c1 - cfg.last_q):c1].float().cpu().numpy(),
                "out": out[:, ri].cpu().numpy(), "lse": lse[:, ri].cpu().numpy(),
                "vs": vs.cpu().numpy(), "ss": ss.cpu().numpy(),
                "verts": [x.numpy() for x in verts], "slashes": [x.numpy() for x in slashes],
                "stats": stats.cpu().tolist(),
            }
    if name == "7b_1m_dca":
        # the same call again on the last chunk: bitwise the same output
        c0, lc = cfg.chunk_bounds(cfg.n_chunks - 1)
        again = torch.empty_like(out[:, :lc])
        lse2 = torch.empty_like(lse[:, :lc])
        layer.attend(q[:, c0:c0 + lc], c0, out=again, lse=lse2)
        res["repeat_equal"] = (bool(torch.equal(again, out[:, :lc])),
                               bool(torch.equal(lse2, lse[:, :lc])))
        del again, lse2
    if name == "14b_256k":
        _dca_twin(cfg, layer, q, k, v, res)
    if name == "14b_512k_refine":
        c0, lc = cfg.chunk_bounds(cfg.n_chunks - 1)
        qc = q[:, c0:c0 + lc]
        rows = np.unique(np.concatenate([
            np.arange(lc - cfg.last_q, lc),
            np.random.default_rng([cfg.seed, 9]).choice(lc, size=64, replace=False)]))
        rows_t = torch.as_tensor(rows.astype(np.int32), device=DEV)
        lf, ls, rc = layer.recall(qc, c0, rows_t)
        verts, slashes = layer.pattern.lists()
        res["recall"] = {"rows": rows + c0, "lse_full": lf.cpu().numpy(),
                         "lse_sparse": ls.cpu().numpy(), "recall": rc.cpu().numpy(),
                         "verts": [x.numpy() for x in verts],
                         "slashes": [x.numpy() for x in slashes],
                         "q": q[:, torch.as_tensor(rows + c0, device=DEV)].float().cpu().numpy()}
        base_v, base_s = list(layer.n_vert), list(layer.n_slash)
        hist = layer.refine_chunk(qc, c0, rows_t, out[:, :lc], lse=lse[:, :lc])
        res["refine"] = {"history": hist, "base": (base_v, base_s),
                         "after": (list(layer.n_vert), list(layer.n_slash)), "c1": c0 + lc}
    if name == "7b_1m_dca":
        # dense mode (every causal key, same DCA logits) on the last chunk
        c0, lc = cfg.chunk_bounds(cfg.n_chunks - 1)
        layer.attend(q[:, c0:c0 + lc], c0, out=out[:, :lc], lse=lse[:, :lc], dense=True)
        rng = np.random.default_rng([cfg.seed, 11])
        rows = np.sort(rng.choice(np.arange(c0, c0 + lc), DENSE_ROWS - 4, replace=False))
        rows = np.unique(np.concatenate([rows, [c0, c0 + 1, c0 + lc // 2, c0 + lc - 1]]))
        ri = torch.as_tensor(rows - c0, device=DEV)
        res["dense"] = {"rows": rows, "out": out[:, ri].cpu().numpy(),
                        "lse": lse[:, ri].cpu().numpy(),
                        "q": q[:, torch.as_tensor(rows, device=DEV)].float().cpu().numpy()}
        # the other head patterns on the last chunk, in buffers of their own:
        # block-sparse with 100 kept blocks and A-shape with sink 16 + window
        # 2048 (the measured configurations)
        c1 = c0 + lc
        oh = group_heads(cfg, cfg.n_chunks - 1)
        rows = sample_rows(cfg, c0, lc)
        ri = torch.as_tensor(rows - c0, device=DEV)
        qr = q[:, torch.as_tensor(rows, device=DEV)].float().cpu().numpy()
        n_qb, n_kb = lc // 64, c1 // 64
        bp = L.BlockPattern(H, n_qb, 100, DEV)
        sc = torch.empty(H, n_qb, n_kb, device=DEV)
        L.block_sparse_estimate(q[:, c0:c1], layer.k_cache[:, :c1], c0, layer.rope, layer.dca,
                                sm, [100] * H, bp, scores=sc)
        st_b = torch.zeros(2, dtype=torch.int64, device=DEV)
        L.block_sparse_attn_prefill(q[:, c0:c1], layer.k_cache[:, :c1], layer.v_cache[:, :c1],
                                    c0, layer.rope, layer.dca, sm, bp, out=out[:, :lc],
                                    lse=lse[:, :lc], stats=st_b)
        res["block"] = {"c0": c0, "rows": rows, "q": qr, "out": out[:, ri].cpu().numpy(),
                        "lse": lse[:, ri].cpu().numpy(), "heads": oh,
                        "idx": {h: bp.idx[h].cpu().numpy() for h in oh},
                        "cnt": {h: bp.cnt[h].cpu().numpy() for h in oh},
                        "scores": {h: sc[h].cpu().numpy() for h in oh},
                        "q_chunk": {h: q[h, c0:c1].float().cpu().numpy() for h in oh},
                        "stats": st_b.cpu().tolist()}
        del sc
        ap = L.Pattern(H, 16, 2048, DEV)
        L.pattern_fill_a_shape(ap, 16, 2048, c1)
        L.vs_sparse_attn_prefill(q[:, c0:c1], layer.k_cache[:, :c1], layer.v_cache[:, :c1], c0,
                                 layer.rope, layer.dca, sm, ap, out=out[:, :lc], lse=lse[:, :lc])
        av, asl = ap.lists()
        res["a_shape"] = {"rows": rows, "q": qr, "out": out[:, ri].cpu().numpy(),
                          "lse": lse[:, ri].cpu().numpy(), "heads": oh,
                          "verts": [x.numpy() for x in av], "slashes": [x.numpy() for x in asl]}
    if name in ("7b_1m_dca", "14b_256k"):
        # decode steps on the full cache: the newest rows (as many as fill the
        # 32 matrix rows, then one) and, with DCA, rows across a period edge
        nmax = 32 // cfg.group
        cases = [(cfg.seq_len - nmax, nmax), (cfg.seq_len - 1, 1)]
        if cfg.dca_chunk:
            S = cfg.dca_chunk - cfg.dca_local
            cases.append((3 * S - 2, min(4, nmax)))
        res["decode"] = []
        for p0, n in cases:
            c1 = p0 + n
            lse_d = torch.empty(H, n, device=DEV)
            od, _ = L.attn_decode(q[:, p0:c1], layer.k_cache[:, :c1], layer.v_cache[:, :c1], p0,
                                  layer.rope, layer.dca, sm, lse=lse_d)
            res["decode"].append({"rows": np.arange(p0, c1), "out": od.cpu().numpy(),
                                  "lse": lse_d.cpu().numpy(),
                                  "q": q[:, p0:c1].float().cpu().numpy()})
    res["k"] = {g: k[g].float().cpu().numpy() for g in range(cfg.n_kv_heads)}
    res["v"] = {g: v[g].float().cpu().numpy() for g in range(cfg.n_kv_heads)}
    del q, k, v, layer, out, lse
    torch.cuda.empty_cache()
    return res


@functools.lru_cache(maxsize=8)
def key_context(name, g, operands="fp64"):
    """fp64 keys and values of KV head g over the whole layer (the oracle only
    reads keys j <= i of each row)."""
    cfg = CONFIGS[name]
    res = run_layer(name)
    return oracle.KeyContext(res["k"][g].astype(np.float64), res["v"][g].astype(np.float64),
                             oracle_freqs(cfg), cfg.dca_chunk, cfg.dca_local, operands=operands)


def warm_contexts(name, groups, cont=False):
    """Build the oracle's rotated keys of these KV heads before forking the
    workers, which then share them."""
    for g in sorted(set(groups)):
        ctx = key_context(name, g)
        ctx.k_dca()
        if cont:
            ctx.k_cont()


def _sparse_job(name, g, q, rows, verts, slashes, sm):
    return oracle.sparse_rows(q, rows, key_context(name, g), verts, slashes, sm)


def _dense_job(name, g, q, rows, sm):
    return oracle.dense_causal_rows(q, rows, key_context(name, g), sm)


def _estimate_job(name, g, q, rows, c1, sm):
    return oracle.estimate_scores(q, rows, key_context(name, g), c1, sm)


def _recall_job(name, g, q, rows, verts, slashes, sm):
    return oracle.attention_recall(q, rows, key_context(name, g), verts, slashes, sm)


def _block_job(name, g, qc, c0, sm):
    return oracle.block_scores(qc, c0, key_context(name, g), sm)


def _block_rows_job(name, g, q, rows, idx, cnt, c0, sm):
    kept = lambda i: idx[(i - c0) // 64, :cnt[(i - c0) // 64]]  # noqa: E731
    return oracle.block_sparse_rows(q, rows, key_context(name, g), kept, sm)


def split_rows(rows, parts):
    """Row index ranges cutting `rows` into about `parts` pieces."""
    edges = np.linspace(0, len(rows), min(parts, len(rows)) + 1).astype(int)
    return [slice(a, b) for a, b in zip(edges[:-1], edges[1:]) if b > a]


NAMES = list(CHECK_CHUNKS)


@pytest.fixture(scope="module", params=NAMES)
def layer_run(request):
    """(name, results): module scope, so the tests are grouped by layer."""
    print(f"[layer] running {request.param} on the GPU", flush=True)
    return request.param, run_layer(request.param)


def test_selection_bit_exact_full_size(layer_run):
    """The selection is the oracle's selection of the same scores: every head
    of every checked chunk."""
    name, res = layer_run
    cfg = CONFIGS[name]
    for c, ch in res["chunks"].items():
        for h in range(cfg.n_heads):
            assert ch["verts"][h].tolist() == \
                oracle.select_top(ch["vs"][h], cfg.n_vert).tolist(), (c, h)
            assert ch["slashes"][h].tolist() == \
                oracle.select_top(ch["ss"][h], cfg.n_slash).tolist(), (c, h)


def test_pair_count_exact_full_size(layer_run):
    """The attention's count of the pairs it weighted (a kernel statistic)
    equals the exact sum of |C_i| over every row and head of each checked
    chunk: the tile walk leaves out no key of any C_i and adds none."""
    name, res = layer_run
    cfg = CONFIGS[name]
    for c, ch in res["chunks"].items():
        c0, c1 = ch["c0"], ch["c0"] + ch["lc"]
        want = sum(critical_pair_total(ch["verts"][h], ch["slashes"][h], c0, c1)
                   for h in range(cfg.n_heads))
        assert ch["stats"][1] == want, (name, c, ch["stats"], want)


def test_estimate_scores_full_size(layer_run):
    """Vertical and slash scores of the last checked chunk against fp64 (one
    head per KV group and the last head); the fp64 top sets differ from the
    GPU's only by near-ties."""
    name, res = layer_run
    cfg = CONFIGS[name]
    c = max(res["chunks"])
    ch = res["chunks"][c]
    c1 = ch["c0"] + ch["lc"]
    rows = oracle.estimate.estimate_rows(ch["c0"], ch["lc"], cfg.last_q)
    heads = sorted(set(group_heads(cfg, c) + [cfg.n_heads - 1]))
    warm_contexts(name, [h // cfg.group for h in heads], cont=True)
    refs = parallel_map(_estimate_job, [(name, h // cfg.group,
                                         ch["q_est"][h].astype(np.float64), rows, c1, res["sm"])
                                        for h in heads], workers=8)
    for h, (rv, rs) in zip(heads, refs):
        gv, gs = ch["vs"][h].astype(np.float64), ch["ss"][h].astype(np.float64)
        n = len(rows)
        assert abs(gv.sum() - n) < 1e-3 * n and abs(gs.sum() - n) < 1e-3 * n
        print(f"[estimate] {name} chunk {c} head {h}:", flush=True)
        rel = SCORE_REL_LARGE_LOGITS if cfg.planting == "far_sinks_stripes" else SCORE_REL
        score_compare(gv, rv, "vertical", rel=rel)
        score_compare(gs, rs, "slash", rel=rel)
        near_tie_check(ch["verts"][h], rv, cfg.n_vert, "vertical")
        near_tie_check(ch["slashes"][h], rs, cfg.n_slash, "slash")


def test_attention_sampled_rows_full_size(layer_run):
    """Sampled rows of every checked chunk against fp64 sparse attention with
    the GPU's pattern: every head on the last checked chunk, one head per KV
    group on the others."""
    name, res = layer_run
    cfg = CONFIGS[name]
    last = max(res["chunks"])
    worst = [0.0, 0.0]
    warm_contexts(name, range(cfg.n_kv_heads))
    for c, ch in res["chunks"].items():
        rows = ch["rows"]
        heads = heads_of_chunk(cfg, c, last)
        refs = parallel_map(_sparse_job, [(name, h // cfg.group, ch["q"][h].astype(np.float64),
                                           rows, ch["verts"][h], ch["slashes"][h], res["sm"])
                                          for h in heads])
        for h, (ro, rl, sizes) in zip(heads, refs):
            print(f"[attention] {name} chunk {c} head {h}: {rows.size} rows, "
                  f"mean |C_i| {sizes.mean():.0f}", flush=True)
            mx, mn = compare(ch["out"][h].astype(np.float64), ro)
            worst = [max(worst[0], mx), max(worst[1], mn)]
            lse_compare(ch["lse"][h].astype(np.float64), rl)
        st = ch["stats"]
        assert st[0] >= st[1] > 0
    # for information: the oracle with fp16-rounded rotated operands (the
    # kernel's own QK^T operand rounding), head 0 of the last chunk
    ch = res["chunks"][last]
    bctx = oracle.KeyContext(key_context(name, 0).K, key_context(name, 0).V,
                             oracle_freqs(cfg), cfg.dca_chunk, cfg.dca_local, operands="fp16")
    sel = slice(0, None, 4)
    bo = oracle.sparse_rows(ch["q"][0][sel].astype(np.float64), ch["rows"][sel], bctx,
                            ch["verts"][0], ch["slashes"][0], res["sm"])[0]
    d = np.abs(ch["out"][0][sel] - bo)
    print(f"[info] {name}: worst vs fp64 max-abs {worst[0]:.2e} mean-abs {worst[1]:.2e}; "
          f"head 0 vs fp16-operand oracle max-abs {d.max():.2e} mean-abs {d.mean():.2e}")


def test_attention_repeat_bitwise():
    """The 1M layer's last chunk attended twice: bitwise the same output and
    lse (no atomics or order-dependent sums in the attention)."""
    res = run_layer("7b_1m_dca")
    assert res["repeat_equal"] == (True, True)


def test_dca_is_identity_within_training_length():
    """14B-shaped 256K layer with DCA on at C = 262,144 (the sequence
    length), W = 32,768: every relative position stays the plain one
    ([Qwen2.5-1M explainer] Length Extrapolation: intra-chunk pairs keep
    their positions, successive pairs inside the window too), so the
    estimate scores and the attention on the same pattern equal the DCA-off
    run to rounding."""
    name = "14b_256k"
    cfg = CONFIGS[name]
    res = run_layer(name)
    # two GPU runs, each within the oracle bars of the exact result: their
    # difference is held to twice those bars
    for c, tw in res["twin"].items():
        ch = res["chunks"][c]
        for h in range(cfg.n_heads):
            score_compare(tw["vs"][h].astype(np.float64), ch["vs"][h].astype(np.float64),
                          "vertical (DCA on vs off)", quiet=True, rel=2 * SCORE_REL)
            score_compare(tw["ss"][h].astype(np.float64), ch["ss"][h].astype(np.float64),
                          "slash (DCA on vs off)", quiet=True, rel=2 * SCORE_REL)
        d = np.abs(tw["out"] - ch["out"])
        print(f"[dca-twin] chunk {c}: DCA on vs off max-abs {d.max():.2e} mean-abs "
              f"{d.mean():.2e}", flush=True)
        compare(tw["out"].astype(np.float64), ch["out"].astype(np.float64), 2 * MAX_ABS,
                2 * MEAN_ABS)
        lse_compare(tw["lse"].astype(np.float64), ch["lse"].astype(np.float64), 4e-2)


def test_recall_and_refinement_full_size():
    """Refinement stress layer: GPU recall against fp64 on sampled rows, the
    calibration rule (some heads under the threshold, some above), and the
    budget decisions of every refinement round."""
    name = "14b_512k_refine"
    cfg = CONFIGS[name]
    res = run_layer(name)
    rc = res["recall"]
    sel = np.linspace(0, rc["rows"].size - 1, RECALL_ROWS).astype(np.int64)
    heads = group_heads(cfg, cfg.n_chunks - 1)
    rows = rc["rows"][sel]
    warm_contexts(name, [h // cfg.group for h in heads])
    refs = parallel_map(_recall_job, [(name, h // cfg.group, rc["q"][h][sel].astype(np.float64),
                                       rows, rc["verts"][h], rc["slashes"][h], res["sm"])
                                      for h in heads])
    for h, (of, os_, orc) in zip(heads, refs):
        lse_compare(rc["lse_full"][h][sel], of)
        lse_compare(rc["lse_sparse"][h][sel], os_)
        assert np.max(np.abs(rc["recall"][h][sel] - orc)) < 1e-2
    hist = res["refine"]["history"]
    mean0 = hist[0]
    print(f"[refine] head recall at the base budget: min {mean0.min():.3f} "
          f"max {mean0.max():.3f}, {int((mean0 < cfg.recall_threshold).sum())} of "
          f"{cfg.n_heads} under {cfg.recall_threshold}")
    assert (mean0 < cfg.recall_threshold).any() and (mean0 >= cfg.recall_threshold).any()
    base_v, base_s = res["refine"]["base"]
    nv, ns, raised = oracle.refine_budgets(mean0, base_v, base_s, res["refine"]["c1"],
                                           cfg.recall_threshold)
    # budgets keep doubling for heads that stay low: replay every round
    for r in range(1, len(hist) - 1):
        nv, ns, more = oracle.refine_budgets(hist[r], nv, ns, res["refine"]["c1"],
                                             cfg.recall_threshold)
    after_v, after_s = res["refine"]["after"]
    assert list(nv) == after_v and list(ns) == after_s
    # larger budgets select supersets of the same scores: recall cannot drop
    assert np.all(hist[1][raised] >= mean0[raised] - 1e-5)


@pytest.mark.timeout(900)
def test_dense_mode_1m_sampled_rows():
    """Dense mode at the 1M context (last chunk): 128 sampled rows, spread
    over the KV groups (a quarter of the rows on one head of each), against
    the oracle's full causal attention with the same DCA logits."""
    name = "7b_1m_dca"
    cfg = CONFIGS[name]
    res = run_layer(name)
    dn = res["dense"]
    n = dn["rows"].size
    warm_contexts(name, range(cfg.n_kv_heads))
    jobs, where = [], []
    for g, h in enumerate(group_heads(cfg, 0)):
        part = slice(g * n // cfg.n_kv_heads, (g + 1) * n // cfg.n_kv_heads)
        sub = np.arange(n)[part]
        for piece in split_rows(sub, 8):
            idx = sub[piece]
            jobs.append((name, g, dn["q"][h][idx].astype(np.float64), dn["rows"][idx], res["sm"]))
            where.append((h, idx))
    refs = parallel_map(_dense_job, jobs)
    for (h, idx), (ro, rl) in zip(where, refs):
        compare(dn["out"][h][idx].astype(np.float64), ro)
        lse_compare(dn["lse"][h][idx].astype(np.float64), rl)
    print(f"[dense] {n} rows over {cfg.n_kv_heads} KV groups", flush=True)


def test_block_sparse_1m_sampled_rows():
    """Block-sparse heads at the 1M context (last chunk, 100 blocks): block
    scores of one head per KV group against fp64, the selection bit-exact on
    the GPU's scores, and sampled rows against the oracle on the GPU's
    lists."""
    name = "7b_1m_dca"
    res = run_layer(name)
    cfg = CONFIGS[name]
    b = res["block"]
    c0 = b["c0"]
    warm_contexts(name, [h // cfg.group for h in b["heads"]], cont=True)
    scores = parallel_map(_block_job, [(name, h // cfg.group,
                                        b["q_chunk"][h].astype(np.float64), c0, res["sm"])
                                       for h in b["heads"]], workers=4)
    rows_ref = parallel_map(_block_rows_job, [(name, h // cfg.group,
                                               b["q"][h].astype(np.float64), b["rows"],
                                               b["idx"][h], b["cnt"][h], c0, res["sm"])
                                              for h in b["heads"]])
    for h, ref, (ro, rl, sizes) in zip(b["heads"], scores, rows_ref):
        got = b["scores"][h].astype(np.float64)
        fin = np.isfinite(ref)
        d = np.abs(got[fin] - ref[fin])
        print(f"[block] {name} head {h}: score max |d| {d.max():.2e} (max |s| "
              f"{np.abs(ref[fin]).max():.2e})", flush=True)
        assert np.all(d <= 1e-3 + 1e-3 * np.abs(ref[fin]))
        idx, cnt = b["idx"][h], b["cnt"][h]
        for qb in range(cnt.size):
            diag = c0 // 64 + qb
            sel = oracle.select_blocks(got[qb, :diag + 1], diag, 100)
            assert cnt[qb] == sel.size and idx[qb, :sel.size].tolist() == sel.tolist(), qb
        compare(b["out"][h].astype(np.float64), ro)
        lse_compare(b["lse"][h].astype(np.float64), rl)
    st = b["stats"]
    assert st[0] >= st[1] > 0


def test_a_shape_1m_sampled_rows():
    """A-shape heads (sink 16, window 2048) at the 1M context: the filled
    lists are the oracle's, and sampled rows of one head per KV group match
    its attention."""
    name = "7b_1m_dca"
    cfg = CONFIGS[name]
    res = run_layer(name)
    a = res["a_shape"]
    ov, os_ = oracle.a_shape_lists(16, 2048, cfg.seq_len)
    for h in range(cfg.n_heads):
        assert a["verts"][h].tolist() == ov.tolist() and a["slashes"][h].tolist() == os_.tolist()
    warm_contexts(name, [h // cfg.group for h in a["heads"]])
    refs = parallel_map(_sparse_job, [(name, h // cfg.group, a["q"][h].astype(np.float64),
                                       a["rows"], ov, os_, res["sm"]) for h in a["heads"]])
    for h, (ro, rl, _) in zip(a["heads"], refs):
        compare(a["out"][h].astype(np.float64), ro)
        lse_compare(a["lse"][h].astype(np.float64), rl)


@pytest.mark.parametrize("name", ["7b_1m_dca", "14b_256k"])
def test_decode_full_size(name):
    """Decode steps over the whole cache (1M keys with DCA and YaRN; 256K with
    5 query heads per KV head) against the oracle's dense causal rows, one
    head per KV group."""
    cfg = CONFIGS[name]
    res = run_layer(name)
    warm_contexts(name, range(cfg.n_kv_heads))
    jobs, where = [], []
    for case in res["decode"]:
        for h in group_heads(cfg, case["rows"][0]):
            jobs.append((name, h // cfg.group, case["q"][h].astype(np.float64), case["rows"],
                         res["sm"]))
            where.append((case, h))
    refs = parallel_map(_dense_job, jobs)
    for (case, h), (ro, rl) in zip(where, refs):
        compare(case["out"][h].astype(np.float64), ro)
        lse_compare(case["lse"][h].astype(np.float64), rl)
