"""The C ABI on a host without a GPU: the library loads, exports every
function include/lcsr.h declares, sizes workspaces, and rejects invalid
arguments with the documented status before it launches anything (every
call below fails validation, so no pointer is ever dereferenced)."""

import ctypes
import os
import re

import pytest

from long_context_sparse_rope_amd import _capi as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # 16-byte aligned stand-in for a device pointer (never read)


def declared_functions():
    text = open(os.path.join(ROOT, "include", "lcsr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(lcsr_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return C.load()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) == 14, names
    assert set(names) == set(C.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def problem(**kw):
    p = C.lcsr_problem_t()
    p.q, p.k_cache, p.v_cache = FAKE, FAKE, FAKE
    p.q_dtype = C.LCSR_BF16
    p.n_heads, p.n_kv_heads, p.head_dim = 28, 4, 128
    p.q_stride_h, p.q_stride_t = 32768 * 128, 128
    p.kv_stride_h, p.kv_stride_t = 1 << 27, 128
    p.chunk_start, p.chunk_len = 32768, 32768
    p.rope.base, p.rope.yarn_factor, p.rope.orig_max_pos = 1e7, 1.0, 262144
    p.rope.beta_fast, p.rope.beta_slow = 32.0, 1.0
    p.sm_scale = 0.0884
    for k, v in kw.items():
        if k.startswith("dca_"):
            setattr(p.dca, k[4:], v)
        else:
            setattr(p, k, v)
    return p


def pattern(max_vert=1000, max_slash=6096):
    t = C.lcsr_pattern_t()
    t.vert_idx = t.vert_cnt = t.slash_idx = t.slash_cnt = FAKE
    t.max_vert, t.max_slash = max_vert, max_slash
    return t


def err(lib):
    return lib.lcsr_last_error().decode()


def test_softmax_scale_yarn_temperature(lib):
    """lcsr_softmax_scale against the closed form worked by hand in
    tests/golden/yarn_temperature.txt (1/t for s = 1, 2, 4) at D 64 and 128,
    and its error returns."""
    path = os.path.join(ROOT, "tests", "golden", "yarn_temperature.txt")
    rows = [[float(x) for x in ln.split()] for ln in open(path)
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 3
    for s, _, inv_t in rows:
        for d in (64, 128):
            r = C.lcsr_rope_t(1e7, s, 262144, 32.0, 1.0, 0)
            got = lib.lcsr_softmax_scale(ctypes.byref(r), d)
            want = inv_t / d ** 0.5
            assert abs(got - want) <= 2 ** -24 * want, (s, d, got, want)
    # s below 1 means no temperature
    r = C.lcsr_rope_t(1e7, 0.5, 262144, 32.0, 1.0, 0)
    assert lib.lcsr_softmax_scale(ctypes.byref(r), 128) == pytest.approx(128 ** -0.5, rel=1e-7)
    assert lib.lcsr_softmax_scale(None, 128) == 0.0 and "rope" in err(lib)
    assert lib.lcsr_softmax_scale(ctypes.byref(r), 0) == 0.0 and "head_dim" in err(lib)
    r.yarn_factor = float("nan")
    assert lib.lcsr_softmax_scale(ctypes.byref(r), 128) == 0.0 and "finite" in err(lib)


def test_workspace_bytes(lib):
    p = problem()
    for which in (C.LCSR_WS_ESTIMATE, C.LCSR_WS_ATTN, C.LCSR_WS_RECALL):
        assert lib.lcsr_workspace_bytes(which, ctypes.byref(p), 1000, 6096) > 0
    # the estimate's workspace grows with the context
    big = problem(chunk_start=1015808)
    assert (lib.lcsr_workspace_bytes(C.LCSR_WS_ESTIMATE, ctypes.byref(big), 1000, 6096) >
            lib.lcsr_workspace_bytes(C.LCSR_WS_ESTIMATE, ctypes.byref(p), 1000, 6096))
    bad = problem(n_kv_heads=3)
    assert lib.lcsr_workspace_bytes(C.LCSR_WS_ATTN, ctypes.byref(bad), 1000, 6096) == 0
    assert "n_kv_heads" in err(lib)
    assert lib.lcsr_workspace_bytes(7, ctypes.byref(p), 1, 1) == 0


def attn(lib, p, pat=None, out=FAKE, out_dtype=C.LCSR_FP32, ws=FAKE, ws_bytes=1 << 40,
         flags=0, o_sh=32768 * 128, o_st=128):
    return lib.lcsr_vs_sparse_attn_prefill(
        ctypes.byref(p), None if pat is None else ctypes.byref(pat), None, out, out_dtype,
        o_sh, o_st, None, None, flags, ws, ws_bytes, None)


@pytest.mark.parametrize("field,value,code,text", [
    ("q", None, C.LCSR_EINVAL, "NULL"),
    ("q", FAKE + 4, C.LCSR_EINVAL, "aligned"),
    ("n_kv_heads", 3, C.LCSR_EINVAL, "multiple"),
    ("head_dim", 96, C.LCSR_ENOTSUP, "head_dim"),
    ("n_heads", 128, C.LCSR_ENOTSUP, "n_heads"),
    ("q_stride_t", 100, C.LCSR_EINVAL, "strides"),
    ("chunk_len", -1, C.LCSR_EINVAL, ">= 0"),
    ("sm_scale", 0.0, C.LCSR_EINVAL, "sm_scale"),
    ("dca_chunk", 262144, C.LCSR_EINVAL, "local"),   # with local = chunk (below)
])
def test_attention_rejects(lib, field, value, code, text):
    kw = {field: value}
    if field == "dca_chunk":
        kw["dca_local"] = 262144          # local must be < chunk
    p = problem(**kw)
    assert attn(lib, p, pattern()) == code
    assert text in err(lib)


def test_attention_rejects_other_arguments(lib):
    p = problem()
    assert attn(lib, p, None) == C.LCSR_EINVAL                      # no pattern, not dense
    assert attn(lib, p, pattern(), out=None) == C.LCSR_EINVAL
    assert attn(lib, p, pattern(), out_dtype=7) == C.LCSR_EINVAL
    assert attn(lib, p, pattern(), o_st=64) == C.LCSR_EINVAL
    need = lib.lcsr_workspace_bytes(C.LCSR_WS_ATTN, ctypes.byref(p), 1000, 6096)
    assert attn(lib, p, pattern(), ws_bytes=need - 1) == C.LCSR_EWORKSPACE
    assert str(need) in err(lib)
    assert attn(lib, p, pattern(), ws=None) == C.LCSR_EWORKSPACE
    # the DCA period must be a multiple of the 32-row block here
    q = problem(dca_chunk=262144, dca_local=32760)
    assert attn(lib, q, pattern()) == C.LCSR_ENOTSUP
    # the context cap (the row block's key bitmap lives in LDS)
    huge = problem(chunk_start=(1 << 30) - 32768)
    assert attn(lib, huge, pattern()) == C.LCSR_ENOTSUP
    assert "contexts up to" in err(lib)


def test_dca_period_alignment_per_call(lib):
    """DCA key periods S = C - W: every call takes S >= 64; the vertical-slash
    attention needs S % 32 == 0 (32-row blocks); the other calls take any S."""
    def ws(which, local):
        p = problem(dca_chunk=262144, dca_local=local)
        return lib.lcsr_workspace_bytes(which, ctypes.byref(p), 1000, 6096)
    s32 = 32736    # S = 229408 = 32 x 7169
    s16 = 32752    # S = 229392 = 16 x 14337
    s4 = 32756     # S = 229388, a multiple of 4 only
    assert ws(C.LCSR_WS_ATTN, s32) > 0
    assert ws(C.LCSR_WS_ATTN, s16) == 0 and ws(C.LCSR_WS_ATTN, s4) == 0
    for which in (C.LCSR_WS_ESTIMATE, C.LCSR_WS_RECALL, C.LCSR_WS_DECODE,
                  C.LCSR_WS_BLOCK_EST, C.LCSR_WS_BLOCK_ATTN):
        assert ws(which, s4) > 0
    # a period below one 64-key tile is refused by every call
    for which in (C.LCSR_WS_ESTIMATE, C.LCSR_WS_ATTN, C.LCSR_WS_DECODE):
        assert ws(which, 262144 - 48) == 0


def test_estimate_and_recall_reject(lib):
    p = problem()
    nv = (ctypes.c_int32 * 28)(*([1000] * 28))
    ns = (ctypes.c_int32 * 28)(*([6096] * 28))
    pat = pattern()

    def est(last_q=64, n_vert=nv, flags=0, vs=None, ws=FAKE, ws_bytes=1 << 40):
        return lib.lcsr_vs_pattern_estimate(ctypes.byref(p), last_q, n_vert, ns, None,
                                            ctypes.byref(pat), vs, None, flags, ws, ws_bytes,
                                            None)

    assert est(last_q=0) == C.LCSR_EINVAL
    assert est(last_q=65) == C.LCSR_EINVAL
    over = (ctypes.c_int32 * 28)(*([1001] + [1000] * 27))
    assert est(n_vert=over) == C.LCSR_EINVAL and "budget" in err(lib)
    assert est(flags=C.LCSR_EST_SELECT_ONLY) == C.LCSR_EINVAL
    assert est(ws_bytes=16) == C.LCSR_EWORKSPACE
    rows = (ctypes.c_int32 * 2)(0, 1)
    assert lib.lcsr_attn_recall_check(ctypes.byref(p), ctypes.byref(pat), None, rows, -1,
                                      FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == C.LCSR_EINVAL
    assert lib.lcsr_attn_recall_check(ctypes.byref(p), ctypes.byref(pat), None, None, 2,
                                      FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == C.LCSR_EINVAL


def test_decode_workspace_and_rejects(lib):
    # decode rows may start anywhere, also with DCA on
    p = problem(chunk_start=1048573, chunk_len=4, dca_chunk=262144, dca_local=32768)
    need = lib.lcsr_workspace_bytes(C.LCSR_WS_DECODE, ctypes.byref(p), 0, 0)
    assert need > 0

    def dec(pp, out=FAKE, out_dtype=C.LCSR_FP32, ws=FAKE, ws_bytes=1 << 40, o_sh=4 * 128,
            o_st=128):
        return lib.lcsr_attn_decode(ctypes.byref(pp), out, out_dtype, o_sh, o_st, None, ws,
                                    ws_bytes, None)

    assert dec(p, ws_bytes=need - 1) == C.LCSR_EWORKSPACE and str(need) in err(lib)
    # 7 heads per KV head x 5 rows > 32 matrix rows
    assert dec(problem(chunk_start=1048573, chunk_len=5)) == C.LCSR_ENOTSUP
    assert "<= 32" in err(lib)
    assert dec(p, out=None) == C.LCSR_EINVAL
    assert dec(p, out_dtype=9) == C.LCSR_EINVAL
    assert dec(p, o_st=64) == C.LCSR_EINVAL
    assert dec(problem(head_dim=96, chunk_len=1)) == C.LCSR_ENOTSUP
    # the prefill keeps its 64-token chunk start with DCA
    q = problem(chunk_start=1048573, chunk_len=4, dca_chunk=262144, dca_local=32768)
    assert attn(lib, q, pattern()) == C.LCSR_ENOTSUP


def test_decode_noalloc_rejects(lib):
    """The no-alloc decode validates like lcsr_attn_decode before it looks up
    its scratch or launches anything (no GPU is touched here)."""
    def dec(pp, out=FAKE, out_dtype=C.LCSR_FP32, o_sh=4 * 128, o_st=128):
        return lib.lcsr_attn_decode_noalloc(ctypes.byref(pp), out, out_dtype, o_sh, o_st, None,
                                            None)

    assert dec(problem(n_kv_heads=3, chunk_len=1)) == C.LCSR_EINVAL
    assert "n_kv_heads" in err(lib)
    # 7 heads per KV head x 5 rows > 32 matrix rows: the decode's own rule
    assert dec(problem(chunk_start=1048573, chunk_len=5)) == C.LCSR_ENOTSUP
    assert "<= 32" in err(lib)
    p = problem(chunk_start=1048573, chunk_len=4, dca_chunk=262144, dca_local=32768)
    assert dec(p, out=None) == C.LCSR_EINVAL
    assert dec(p, out_dtype=9) == C.LCSR_EINVAL
    assert dec(problem(head_dim=96, chunk_len=1)) == C.LCSR_ENOTSUP
    # the largest problem the decode accepts fits the 8 MiB scratch: 64 KV
    # heads of one query head, 32 rows each, head_dim 128, a 1M-token cache
    big = problem(n_heads=64, n_kv_heads=64, chunk_start=1 << 20, chunk_len=32)
    assert 0 < lib.lcsr_workspace_bytes(C.LCSR_WS_DECODE, ctypes.byref(big), 0, 0) <= 8 << 20
    big = problem(n_heads=64, n_kv_heads=4, chunk_start=1 << 20, chunk_len=2)
    assert 0 < lib.lcsr_workspace_bytes(C.LCSR_WS_DECODE, ctypes.byref(big), 0, 0) <= 8 << 20


def test_fill_a_shape_rejects(lib):
    """Every rejection happens before a launch (nothing is written)."""
    def fill(pat, n_heads=28, mask=None, n_sink=16, n_local=2048, n_ctx=65536):
        return lib.lcsr_pattern_fill_a_shape(
            None if pat is None else ctypes.byref(pat), n_heads, mask, n_sink, n_local, n_ctx,
            None)

    assert fill(None) == C.LCSR_EINVAL
    assert fill(pattern(), n_heads=0) == C.LCSR_EINVAL
    assert fill(pattern(), n_heads=65) == C.LCSR_EINVAL
    assert fill(pattern(), n_sink=-1) == C.LCSR_EINVAL
    assert fill(pattern(), n_ctx=-5) == C.LCSR_EINVAL
    assert fill(pattern(max_vert=8), n_sink=9) == C.LCSR_EINVAL and "max_vert" in err(lib)
    assert fill(pattern(max_slash=100), n_local=101) == C.LCSR_EINVAL
    bad = pattern()
    bad.slash_cnt = None
    assert fill(bad) == C.LCSR_EINVAL
    # a mask that selects no head launches nothing and succeeds
    none = (ctypes.c_int32 * 28)()
    assert fill(pattern(), mask=none) == C.LCSR_OK


def test_block_sparse_rejects(lib):
    """Rejections before any launch (nothing written): alignment, budgets,
    NULL arrays, workspace, context limit."""
    p = problem()
    need_e = lib.lcsr_workspace_bytes(C.LCSR_WS_BLOCK_EST, ctypes.byref(p), 0, 0)
    need_a = lib.lcsr_workspace_bytes(C.LCSR_WS_BLOCK_ATTN, ctypes.byref(p), 0, 0)
    # pooled keys + pooled queries + scores (28 x 512 x 1024 fp32 alone);
    # the attention holds at least one rotated copy of the chunk's queries
    assert need_e > 28 * 512 * 1024 * 4
    assert need_a >= 28 * 32768 * 128 * 2
    budgets = (ctypes.c_int32 * 28)(*([8] * 28))

    def est(pp, nb=budgets, max_blocks=16, idx=FAKE, cnt=FAKE, scores=None, flags=0,
            ws=FAKE, ws_bytes=1 << 40):
        return lib.lcsr_block_sparse_estimate(ctypes.byref(pp), nb, None, max_blocks, idx, cnt,
                                              scores, flags, ws, ws_bytes, None)

    def att(pp, max_blocks=16, idx=FAKE, cnt=FAKE, out=FAKE, out_dtype=C.LCSR_FP32,
            ws=FAKE, ws_bytes=1 << 40):
        return lib.lcsr_block_sparse_attn_prefill(ctypes.byref(pp), idx, cnt, max_blocks, None,
                                                  out, out_dtype, 128, 128 * 32768, None, None,
                                                  ws, ws_bytes, None)

    assert est(problem(chunk_start=32768 + 32)) == C.LCSR_EINVAL and "% 64" in err(lib)
    assert est(p, max_blocks=0) == C.LCSR_EINVAL
    assert est(p, max_blocks=4) == C.LCSR_EINVAL and "n_blocks[0]" in err(lib)
    assert est(p, nb=None) == C.LCSR_EINVAL
    assert est(p, idx=None) == C.LCSR_EINVAL
    assert est(p, flags=C.LCSR_BS_SELECT_ONLY) == C.LCSR_EINVAL
    assert est(p, ws_bytes=need_e - 1) == C.LCSR_EWORKSPACE
    far = problem(chunk_start=1 << 21, chunk_len=64)
    assert est(far) == C.LCSR_ENOTSUP and "key blocks" in err(lib)
    assert att(problem(chunk_start=32768 + 32)) == C.LCSR_EINVAL
    assert att(p, cnt=None) == C.LCSR_EINVAL
    assert att(p, out=None) == C.LCSR_EINVAL
    assert att(p, out_dtype=7) == C.LCSR_EINVAL
    assert att(p, ws_bytes=need_a - 1) == C.LCSR_EWORKSPACE
    assert att(problem(head_dim=96)) == C.LCSR_ENOTSUP


def test_rope_and_dca_reject(lib):
    rope = C.lcsr_rope_t(1e4, 1.0, 262144, 32.0, 1.0, 0)
    call = lib.lcsr_rope_yarn_apply
    ok = dict(x=FAKE, x_dtype=C.LCSR_BF16, xsh=1024 * 64, xst=64, y=2 * FAKE, ysh=1024 * 64,
              yst=64, nh=1, nt=1024, hd=64, pos=FAKE)

    def r(**kw):
        a = dict(ok, **kw)
        return call(a["x"], a["x_dtype"], a["xsh"], a["xst"], a["y"], a["ysh"], a["yst"], a["nh"],
                    a["nt"], a["hd"], a["pos"], ctypes.byref(rope), 1.0, 0, None)

    assert r(x=None) == C.LCSR_EINVAL
    assert r(pos=None) == C.LCSR_EINVAL
    assert r(hd=63) == C.LCSR_EINVAL
    assert r(hd=512) == C.LCSR_EINVAL
    assert r(x_dtype=5) == C.LCSR_EINVAL
    assert r(nt=-1) == C.LCSR_EINVAL
    dca = C.lcsr_dca_t(256, 256)
    assert lib.lcsr_dca_positions(0, 16, ctypes.byref(dca), FAKE, None, None, None,
                                  None) == C.LCSR_EINVAL
    dca = C.lcsr_dca_t(256, 64)
    assert lib.lcsr_dca_positions(0, -1, ctypes.byref(dca), FAKE, None, None, None,
                                  None) == C.LCSR_EINVAL


def test_binding_checks_lse_layout():
    """lse crosses the ABI without strides: the binding takes only a dense
    float32 [H, rows] block (a column slice of a wider buffer is refused)."""
    import torch
    from long_context_sparse_rope_amd.ops import _dense_rows
    whole = torch.zeros(4, 10)
    assert _dense_rows(None, 4, 5, "lse") is None
    assert _dense_rows(whole[:, :5].contiguous(), 4, 5, "lse") is not None
    for bad in (whole[:, :5], whole, torch.zeros(4, 5, dtype=torch.float64)):
        with pytest.raises(ValueError):
            _dense_rows(bad, 4, 5, "lse")
