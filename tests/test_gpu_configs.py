"""Parity at the full layer shapes, on sampled outputs.

Each layer (7B-shaped 128K, 14B-shaped 256K, 7B-shaped 1M with DCA and
YaRN s = 4, 14B-shaped 512K refinement stress) runs its whole chunk loop on
the GPU through the C ABI, in the launch configuration the benchmark times.
For a few chunks per layer (the first, the ones that straddle a DCA key
period or the local window, the last) the run keeps:

* the estimate scores of every head, so that the selection can be checked
  bit for bit against the oracle's selection of the same fp32 scores;
* the attention output and lse of sampled rows: the chunk's estimate rows,
  its first rows, rows beside each DCA period edge (S k +- 2) and beside the
  local-window edge (S k + W - 1, S k + W), and 128 seeded rows.

Three query heads per layer (the first, the last of the first KV group and
the last head) are recomputed by the fp64 oracle: estimate scores of the
last checked chunk, and attention of the sampled rows with the GPU's own
pattern.  Every chunk's full output is checked to be finite.
"""

import functools

import numpy as np
import pytest
import torch

import long_context_sparse_rope_amd as L
import oracle
import synth
from synth.configs import CONFIGS
from tests.gpu_util import DEV, compare, dca_of, lse_compare, oracle_freqs, rope_of

pytestmark = pytest.mark.gpu

CHECK_CHUNKS = {
    "7b_128k": (0, 3),
    "14b_256k": (0, 7),
    "7b_1m_dca": (7, 8, 31),
    "14b_512k_refine": (7, 8, 15),
}
N_SEEDED_ROWS = 128
RECALL_ROWS = 16  # rows per oracle head in the recall check


def oracle_heads(cfg):
    return sorted({0, cfg.group - 1, cfg.n_heads - 1})


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


@functools.lru_cache(maxsize=2)
def run_layer(name):
    """Run the layer's chunk loop on the GPU; keep what the checks need."""
    cfg = CONFIGS[name]
    torch.cuda.empty_cache()
    q, k, v = synth.generate(cfg, DEV)
    sm = oracle.softmax_scale(cfg.head_dim, cfg.yarn_factor)
    H, D = cfg.n_heads, cfg.head_dim
    layer = L.ChunkedSparsePrefill(H, cfg.n_kv_heads, D, cfg.seq_len, rope_of(cfg),
                                   dca_of(cfg), sm, cfg.n_vert, cfg.n_slash, cfg.last_q, DEV)
    res = {"chunks": {}, "sm": sm}
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
        res["refine"] = {"history": [h.numpy() for h in hist], "base": (base_v, base_s),
                         "after": (list(layer.n_vert), list(layer.n_slash)), "c1": c0 + lc}
    if name == "7b_1m_dca":
        # dense mode (every causal key, same DCA logits) on the last chunk
        c0, lc = cfg.chunk_bounds(cfg.n_chunks - 1)
        layer.attend(q[:, c0:c0 + lc], c0, out=out[:, :lc], lse=lse[:, :lc], dense=True)
        rows = np.array([c0, c0 + 1, c0 + lc // 2, c0 + lc - 1], dtype=np.int64)
        ri = torch.as_tensor(rows - c0, device=DEV)
        res["dense"] = {"rows": rows, "out": out[:, ri].cpu().numpy(),
                        "lse": lse[:, ri].cpu().numpy(),
                        "q": q[:, torch.as_tensor(rows, device=DEV)].float().cpu().numpy()}
        # the other head patterns on the last chunk, in buffers of their own:
        # block-sparse with 100 kept blocks and A-shape with sink 16 + window
        # 2048 (the measured configurations)
        c1 = c0 + lc
        oh = oracle_heads(cfg)
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
                        "lse": lse[:, ri].cpu().numpy(),
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
                          "lse": lse[:, ri].cpu().numpy(),
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
    kv_heads = sorted({h // cfg.group for h in oracle_heads(cfg)})
    res["k"] = {g: k[g].float().cpu().numpy() for g in kv_heads}
    res["v"] = {g: v[g].float().cpu().numpy() for g in kv_heads}
    del q, k, v, layer, out, lse
    torch.cuda.empty_cache()
    return res


@functools.lru_cache(maxsize=2)
def key_context(name, g):
    """fp64 keys and values of KV head g over the whole layer (the oracle only
    reads keys j <= i of each row)."""
    cfg = CONFIGS[name]
    res = run_layer(name)
    return oracle.KeyContext(res["k"][g].astype(np.float64), res["v"][g].astype(np.float64),
                             oracle_freqs(cfg), cfg.dca_chunk, cfg.dca_local, operands="bf16")


NAMES = list(CHECK_CHUNKS)


@pytest.fixture(scope="module", params=NAMES)
def layer_run(request):
    """(name, results): module scope, so the tests are grouped by layer."""
    print(f"[layer] running {request.param} on the GPU", flush=True)
    return request.param, run_layer(request.param)


def test_selection_bit_exact_full_size(layer_run):
    """The selection is the oracle's selection of the same scores: every head
    in the last chunk, the oracle heads in the others."""
    name, res = layer_run
    cfg = CONFIGS[name]
    last = max(res["chunks"])
    for c, ch in res["chunks"].items():
        for h in (range(cfg.n_heads) if c == last else oracle_heads(cfg)):
            assert ch["verts"][h].tolist() == \
                oracle.select_top(ch["vs"][h], cfg.n_vert).tolist(), (c, h)
            assert ch["slashes"][h].tolist() == \
                oracle.select_top(ch["ss"][h], cfg.n_slash).tolist(), (c, h)


def test_estimate_scores_full_size(layer_run):
    """Vertical and slash scores of the last checked chunk against fp64."""
    name, res = layer_run
    cfg = CONFIGS[name]
    c = max(res["chunks"])
    ch = res["chunks"][c]
    c1 = ch["c0"] + ch["lc"]
    rows = oracle.estimate.estimate_rows(ch["c0"], ch["lc"], cfg.last_q)
    for h in oracle_heads(cfg):
        ctx = key_context(name, h // cfg.group)
        rv, rs = oracle.estimate_scores(ch["q_est"][h].astype(np.float64), rows, ctx, c1,
                                        res["sm"])
        gv, gs = ch["vs"][h].astype(np.float64), ch["ss"][h].astype(np.float64)
        n = len(rows)
        assert abs(gv.sum() - n) < 1e-3 * n and abs(gs.sum() - n) < 1e-3 * n
        dv, ds = np.max(np.abs(gv - rv)), np.max(np.abs(gs - rs))
        print(f"[estimate] {name} chunk {c} head {h}: max |dv| {dv:.2e} (max v {rv.max():.2e})"
              f" max |ds| {ds:.2e} (max s {rs.max():.2e})")
        assert dv <= 2e-2 * rv.max() and ds <= 2e-2 * rs.max()
        # the fp64 top sets differ from the GPU's only by near-ties
        ov = set(oracle.select_top(rv, cfg.n_vert).tolist())
        os_ = set(oracle.select_top(rs, cfg.n_slash).tolist())
        assert len(ov & set(ch["verts"][h].tolist())) >= 0.9 * len(ov)
        assert len(os_ & set(ch["slashes"][h].tolist())) >= 0.9 * len(os_)


def test_attention_sampled_rows_full_size(layer_run):
    """Sampled rows of every checked chunk against fp64 sparse attention with
    the GPU's pattern."""
    name, res = layer_run
    cfg = CONFIGS[name]
    for c, ch in res["chunks"].items():
        c1 = ch["c0"] + ch["lc"]
        rows = ch["rows"]
        for h in oracle_heads(cfg):
            ctx = key_context(name, h // cfg.group)
            ro, rl, sizes = oracle.sparse_rows(ch["q"][h].astype(np.float64), rows, ctx,
                                               ch["verts"][h], ch["slashes"][h], res["sm"])
            print(f"[attention] {name} chunk {c} head {h}: {rows.size} rows, "
                  f"mean |C_i| {sizes.mean():.0f}")
            compare(ch["out"][h].astype(np.float64), ro)
            lse_compare(ch["lse"][h].astype(np.float64), rl)
            if h == 0:
                # for information: against exact (fp64) rotated operands
                ex = oracle.KeyContext(ctx.K, ctx.V, ctx.inv_freq, ctx.dca_chunk,
                                       ctx.dca_local)
                sel = slice(0, None, 4)
                eo = oracle.sparse_rows(ch["q"][h][sel].astype(np.float64), rows[sel], ex,
                                        ch["verts"][h], ch["slashes"][h], res["sm"])[0]
                d = np.abs(ch["out"][h][sel] - eo)
                print(f"[info] {name} chunk {c} head 0 vs exact operands: max-abs {d.max():.2e}"
                      f" mean-abs {d.mean():.2e}")
        st = ch["stats"]
        assert st[0] >= st[1] > 0


def test_recall_and_refinement_full_size():
    """Refinement stress layer: GPU recall against fp64 on sampled rows, the
    calibration rule (some heads under the threshold, some above), and the
    budget decisions of one refinement round."""
    name = "14b_512k_refine"
    cfg = CONFIGS[name]
    res = run_layer(name)
    rc = res["recall"]
    c1 = res["refine"]["c1"]
    sel = np.linspace(0, rc["rows"].size - 1, RECALL_ROWS).astype(np.int64)
    for h in oracle_heads(cfg):
        ctx = key_context(name, h // cfg.group)
        rows = rc["rows"][sel]
        of, os_, orc = oracle.attention_recall(rc["q"][h][sel].astype(np.float64), rows, ctx,
                                               rc["verts"][h], rc["slashes"][h], res["sm"])
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
    nv, ns, raised = oracle.refine_budgets(mean0, base_v, base_s, c1, cfg.recall_threshold)
    # budgets keep doubling for heads that stay low: replay every round
    for r in range(1, len(hist) - 1):
        nv, ns, more = oracle.refine_budgets(hist[r], nv, ns, c1, cfg.recall_threshold)
    after_v, after_s = res["refine"]["after"]
    assert list(nv) == after_v and list(ns) == after_s
    # larger budgets select supersets of the same scores: recall cannot drop
    assert np.all(hist[1][raised] >= mean0[raised] - 1e-5)


def test_dense_mode_1m_sampled_rows():
    """Dense mode at the 1M context (last chunk): sampled rows against the
    oracle's full causal attention with the same DCA logits."""
    name = "7b_1m_dca"
    cfg = CONFIGS[name]
    res = run_layer(name)
    dn = res["dense"]
    for h in (0, cfg.n_heads - 1):
        ctx = key_context(name, h // cfg.group)
        ro, rl = oracle.dense_causal_rows(dn["q"][h].astype(np.float64), dn["rows"], ctx,
                                          res["sm"])
        compare(dn["out"][h].astype(np.float64), ro)
        lse_compare(dn["lse"][h].astype(np.float64), rl)


def test_block_sparse_1m_sampled_rows():
    """Block-sparse heads at the 1M context (last chunk, 100 blocks): block
    scores of the oracle heads against fp64, the selection bit-exact on the
    GPU's scores, and sampled rows against the oracle on the GPU's lists."""
    name = "7b_1m_dca"
    cfg = CONFIGS[name]
    res = run_layer(name)
    b = res["block"]
    c0 = b["c0"]
    for h in oracle_heads(cfg):
        ctx = key_context(name, h // cfg.group)
        ref = oracle.block_scores(b["q_chunk"][h].astype(np.float64), c0, ctx, res["sm"])
        got = b["scores"][h].astype(np.float64)
        fin = np.isfinite(ref)
        d = np.abs(got[fin] - ref[fin])
        print(f"[block] {name} head {h}: score max |d| {d.max():.2e} (max |s| "
              f"{np.abs(ref[fin]).max():.2e})", flush=True)
        assert np.all(d <= 1e-4 + 1e-4 * np.abs(ref[fin]))
        idx, cnt = b["idx"][h], b["cnt"][h]
        for qb in range(cnt.size):
            diag = c0 // 64 + qb
            sel = oracle.select_blocks(got[qb, :diag + 1], diag, 100)
            assert cnt[qb] == sel.size and idx[qb, :sel.size].tolist() == sel.tolist(), qb
        kept = lambda i: idx[(i - c0) // 64, :cnt[(i - c0) // 64]]  # noqa: E731
        ro, rl, sizes = oracle.block_sparse_rows(b["q"][h].astype(np.float64), b["rows"], ctx,
                                                 kept, res["sm"])
        compare(b["out"][h].astype(np.float64), ro)
        lse_compare(b["lse"][h].astype(np.float64), rl)
    st = b["stats"]
    assert st[0] >= st[1] > 0


def test_a_shape_1m_sampled_rows():
    """A-shape heads (sink 16, window 2048) at the 1M context: the filled
    lists are the oracle's, and sampled rows match its attention."""
    name = "7b_1m_dca"
    cfg = CONFIGS[name]
    res = run_layer(name)
    a = res["a_shape"]
    ov, os_ = oracle.a_shape_lists(16, 2048, cfg.seq_len)
    for h in range(cfg.n_heads):
        assert a["verts"][h].tolist() == ov.tolist() and a["slashes"][h].tolist() == os_.tolist()
    for h in oracle_heads(cfg):
        ctx = key_context(name, h // cfg.group)
        ro, rl, _ = oracle.sparse_rows(a["q"][h].astype(np.float64), a["rows"], ctx, ov, os_,
                                       res["sm"])
        compare(a["out"][h].astype(np.float64), ro)
        lse_compare(a["lse"][h].astype(np.float64), rl)


@pytest.mark.parametrize("name", ["7b_1m_dca", "14b_256k"])
def test_decode_full_size(name):
    """Decode steps over the whole cache (1M keys with DCA and YaRN; 256K with
    5 query heads per KV head) against the oracle's dense causal rows."""
    cfg = CONFIGS[name]
    res = run_layer(name)
    for case in res["decode"]:
        for h in oracle_heads(cfg):
            ctx = key_context(name, h // cfg.group)
            ro, rl = oracle.dense_causal_rows(case["q"][h].astype(np.float64), case["rows"],
                                              ctx, res["sm"])
            compare(case["out"][h].astype(np.float64), ro)
            lse_compare(case["lse"][h].astype(np.float64), rl)
