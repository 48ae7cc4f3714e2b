"""Thin Python binding of the C-ABI calls (argument marshalling only).

Each function has the name of its C entry point without the ``lcsr_``
prefix.  Tensors are torch device tensors (PyTorch supplies device memory
and the stream); every computation runs in liblcsr.so.

Workspaces: a call without a ``workspace`` argument uses one buffer per
call kind and device, cached here and grown on demand.  Calls of the same
kind that may overlap (on different streams) must each pass a workspace of
their own (sized with ``workspace_bytes``); calls on one stream are ordered
and can share the cached one.
"""

import ctypes
from dataclasses import dataclass

import torch

from . import _capi as C


class LcsrError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"lcsr error {code}: {msg}")
        self.code = code


@dataclass(frozen=True)
class RopeConfig:
    """RoPE base and YaRN settings (lcsr_rope_t)."""
    base: float = 1e4
    yarn_factor: float = 1.0
    orig_max_pos: int = 262144
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    freq_blend: bool = False

    def c(self):
        return C.lcsr_rope_t(self.base, self.yarn_factor, self.orig_max_pos, self.beta_fast,
                             self.beta_slow, C.LCSR_ROPE_YARN_FREQ if self.freq_blend else 0)


@dataclass(frozen=True)
class DcaConfig:
    """Dual Chunk Attention: chunk = C (0: off), local = W (lcsr_dca_t)."""
    chunk: int = 0
    local: int = 0

    def c(self):
        return C.lcsr_dca_t(self.chunk, self.local)


def softmax_scale(head_dim, rope):
    """The attention calls' logit scale 1 / (t sqrt(D)), YaRN temperature
    from rope.yarn_factor (lcsr_softmax_scale)."""
    r = rope.c()
    v = C.load().lcsr_softmax_scale(ctypes.byref(r), int(head_dim))
    if not v > 0.0:
        _check(C.LCSR_EINVAL)
    return v


class Pattern:
    """Device buffers of a vertical-slash pattern (lcsr_pattern_t)."""

    def __init__(self, n_heads, max_vert, max_slash, device):
        self.max_vert = int(max_vert)
        self.max_slash = int(max_slash)
        self.vert_idx = torch.full((n_heads, max(1, self.max_vert)), -1, dtype=torch.int32,
                                   device=device)
        self.slash_idx = torch.full((n_heads, max(1, self.max_slash)), -1, dtype=torch.int32,
                                    device=device)
        self.vert_cnt = torch.zeros(n_heads, dtype=torch.int32, device=device)
        self.slash_cnt = torch.zeros(n_heads, dtype=torch.int32, device=device)

    @classmethod
    def from_lists(cls, verts, slashes, device, max_vert=None, max_slash=None):
        """Pattern from per-head index lists (host), sorted ascending."""
        H = len(verts)
        mv = max_vert or max(1, max(len(v) for v in verts))
        ms = max_slash or max(1, max(len(s) for s in slashes))
        p = cls(H, mv, ms, device)
        for h in range(H):
            v = torch.as_tensor(sorted(int(x) for x in verts[h]), dtype=torch.int32)
            s = torch.as_tensor(sorted(int(x) for x in slashes[h]), dtype=torch.int32)
            p.vert_idx[h, :len(v)] = v.to(device)
            p.slash_idx[h, :len(s)] = s.to(device)
            p.vert_cnt[h] = len(v)
            p.slash_cnt[h] = len(s)
        return p

    def c(self):
        return C.lcsr_pattern_t(self.vert_idx.data_ptr(), self.vert_cnt.data_ptr(),
                                self.max_vert, self.slash_idx.data_ptr(),
                                self.slash_cnt.data_ptr(), self.max_slash)

    def lists(self):
        """Per-head (verticals, slashes) as host int64 tensors."""
        vi, vc = self.vert_idx.cpu(), self.vert_cnt.cpu()
        si, sc = self.slash_idx.cpu(), self.slash_cnt.cpu()
        return ([vi[h, :vc[h]].long() for h in range(vi.shape[0])],
                [si[h, :sc[h]].long() for h in range(si.shape[0])])


class BlockPattern:
    """Device buffers of a block-sparse pattern for one chunk: kept key
    blocks idx [H, n_qb, max_blocks] (ascending, -1 padded) and counts
    cnt [H, n_qb]; n_qb = ceil(chunk_len / 64)."""

    def __init__(self, n_heads, n_qb, max_blocks, device):
        self.max_blocks = int(max_blocks)
        self.idx = torch.full((n_heads, max(1, n_qb), self.max_blocks), -1, dtype=torch.int32,
                              device=device)
        self.cnt = torch.zeros((n_heads, max(1, n_qb)), dtype=torch.int32, device=device)


def _check(rc):
    if rc != 0:
        raise LcsrError(rc, C.load().lcsr_last_error().decode())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return C.LCSR_BF16
    if t.dtype == torch.float32:
        return C.LCSR_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _host_i32(values):
    """Host int32 array for a (host) pointer argument, kept alive by the caller."""
    return (ctypes.c_int32 * len(values))(*[int(x) for x in values])


def _ptr(arr):
    return None if arr is None else ctypes.cast(arr, ctypes.c_void_p)


def _head_mask(mask, H):
    if mask is None:
        return None
    if len(mask) != H:
        raise ValueError("head_mask needs one entry per query head")
    return _host_i32([bool(x) for x in mask])


def _dense_rows(t, H, n, what):
    """A per-(head, row) fp32 output must be one dense [H, n] block: the C
    ABI takes it without strides."""
    if t is None:
        return None
    if (t.dtype != torch.float32 or tuple(t.shape) != (H, n) or not t.is_contiguous()):
        raise ValueError(f"{what} must be a contiguous float32 tensor of shape [{H}, {n}]")
    return t.data_ptr()


def _problem(q, k_cache, v_cache, chunk_start, rope, dca, sm_scale):
    if q.dim() != 3 or k_cache.dim() != 3:
        raise ValueError("q is [H, L, D], caches are [H_kv, N, D]")
    if q.stride(2) != 1 or k_cache.stride(2) != 1 or (v_cache is not None and v_cache.stride(2) != 1):
        raise ValueError("the head dimension must be contiguous")
    if k_cache.dtype != torch.float16 or (v_cache is not None and v_cache.dtype != torch.bfloat16):
        raise TypeError("the K cache must be float16 and the V cache bfloat16")
    if v_cache is not None and v_cache.stride() != k_cache.stride():
        raise ValueError("K and V caches must share strides")
    H, L, D = q.shape
    return C.lcsr_problem_t(
        q.data_ptr(), _dtype_code(q), q.stride(0), q.stride(1),
        k_cache.data_ptr(), 0 if v_cache is None else v_cache.data_ptr(),
        k_cache.stride(0), k_cache.stride(1), H, k_cache.shape[0], D,
        int(chunk_start), L, rope.c(), dca.c(), float(sm_scale))


_ws_cache = {}


def _workspace(kind, prob, max_vert, max_slash, device, workspace):
    nbytes = C.load().lcsr_workspace_bytes(kind, ctypes.byref(prob), max_vert, max_slash)
    if nbytes == 0:
        _check(C.LCSR_EINVAL)
    if workspace is not None:
        return workspace
    key = (kind, str(device))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(int(nbytes), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def workspace_bytes(kind, q, k_cache, chunk_start, rope, dca, sm_scale=1.0, max_vert=0,
                    max_slash=0):
    prob = _problem(q, k_cache, None, chunk_start, rope, dca, sm_scale)
    return C.load().lcsr_workspace_bytes(kind, ctypes.byref(prob), max_vert, max_slash)


def rope_yarn_apply(x, pos, rope, out=None, scale=1.0, rotate=True, out_dtype=torch.bfloat16,
                    stream=None):
    """out[h, t] = scale * R(pos[t]) x[h, t] stored bf16 or fp16 (the dtype of
    `out`, else out_dtype) (lcsr_rope_yarn_apply)."""
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("x must be [H, n, D] with a contiguous last dimension")
    H, n, D = x.shape
    if out is None:
        out = torch.empty((H, n, D), dtype=out_dtype, device=x.device)
    if (out.dtype not in (torch.bfloat16, torch.float16) or out.shape != x.shape
            or out.stride(2) != 1):
        raise ValueError("out must be bf16 or fp16 with the shape of x")
    flags = 0 if rotate else C.LCSR_ROPE_NO_ROTATE
    if out.dtype == torch.float16:
        flags |= C.LCSR_ROPE_OUT_FP16
    r = rope.c()
    _check(C.load().lcsr_rope_yarn_apply(
        x.data_ptr(), _dtype_code(x), x.stride(0), x.stride(1), out.data_ptr(), out.stride(0),
        out.stride(1), H, n, D, None if pos is None else pos.data_ptr(), ctypes.byref(r),
        float(scale), flags, _stream(stream)))
    return out


def dca_positions(tok_start, n_tok, dca, device, stream=None):
    """DCA position maps {pk, intra, succ, inter} as int32 tensors."""
    outs = {k: torch.empty(n_tok, dtype=torch.int32, device=device)
            for k in ("pk", "intra", "succ", "inter")}
    d = dca.c()
    _check(C.load().lcsr_dca_positions(int(tok_start), int(n_tok), ctypes.byref(d),
                                       outs["pk"].data_ptr(), outs["intra"].data_ptr(),
                                       outs["succ"].data_ptr(), outs["inter"].data_ptr(),
                                       _stream(stream)))
    return outs


def pattern_fill_a_shape(pattern, n_sink, n_local, n_ctx, head_mask=None, stream=None):
    """Write the A-shape (verticals 0 .. n_sink - 1, slashes 0 .. n_local - 1,
    cut at n_ctx) into the rows of `pattern` selected by head_mask
    (lcsr_pattern_fill_a_shape); other rows are left as they are."""
    H = pattern.vert_cnt.shape[0]
    hm = _head_mask(head_mask, H)
    pat = pattern.c()
    _check(C.load().lcsr_pattern_fill_a_shape(ctypes.byref(pat), H, _ptr(hm), int(n_sink),
                                               int(n_local), int(n_ctx), _stream(stream)))
    return pattern


def block_sparse_estimate(q, k_cache, chunk_start, rope, dca, sm_scale, n_blocks, pattern,
                          head_mask=None, scores=None, select_only=False, workspace=None,
                          stream=None):
    """Fill the BlockPattern `pattern` with each query block's kept key
    blocks (lcsr_block_sparse_estimate); `scores` fp32 [H, n_qb, n_kb] is
    written if given (an input with select_only)."""
    prob = _problem(q, k_cache, None, chunk_start, rope, dca, sm_scale)
    H, n = q.shape[0], q.shape[1]
    if len(n_blocks) != H:
        raise ValueError("one budget per query head")
    n_qb = -(-n // 64)
    if pattern.idx.shape[0] != H or pattern.idx.shape[1] < n_qb:
        raise ValueError("pattern buffers too small for this chunk")
    if scores is not None:
        n_kb = -(-(chunk_start + n) // 64)
        if (scores.dtype != torch.float32 or tuple(scores.shape) != (H, n_qb, n_kb)
                or not scores.is_contiguous()):
            raise ValueError(f"scores must be contiguous float32 [{H}, {n_qb}, {n_kb}]")
    nb = _host_i32(n_blocks)
    hm = _head_mask(head_mask, H)
    if select_only:
        ws = torch.empty(16, dtype=torch.uint8, device=q.device)
    else:
        ws = _workspace(C.LCSR_WS_BLOCK_EST, prob, 0, 0, q.device, workspace)
    idx, cnt = pattern.idx[:, :n_qb], pattern.cnt[:, :n_qb]
    if not (idx.is_contiguous() and cnt.is_contiguous()):
        raise ValueError("pattern buffers must hold exactly this chunk's query blocks")
    _check(C.load().lcsr_block_sparse_estimate(
        ctypes.byref(prob), _ptr(nb), _ptr(hm), pattern.max_blocks, idx.data_ptr(),
        cnt.data_ptr(), None if scores is None else scores.data_ptr(),
        C.LCSR_BS_SELECT_ONLY if select_only else 0, ws.data_ptr(), ws.numel(), _stream(stream)))
    return pattern


def block_sparse_attn_prefill(q, k_cache, v_cache, chunk_start, rope, dca, sm_scale, pattern,
                              out=None, out_dtype=torch.float32, lse=None, stats=None,
                              head_mask=None, workspace=None, stream=None):
    """Attention of the chunk's rows over their kept key blocks
    (lcsr_block_sparse_attn_prefill).  Returns (out [H, L, D], lse or None)."""
    prob = _problem(q, k_cache, v_cache, chunk_start, rope, dca, sm_scale)
    H, n, D = q.shape
    n_qb = -(-n // 64)
    if out is None:
        out = torch.empty((H, n, D), dtype=out_dtype, device=q.device)
    idx, cnt = pattern.idx[:, :n_qb], pattern.cnt[:, :n_qb]
    if not (idx.is_contiguous() and cnt.is_contiguous()):
        raise ValueError("pattern buffers must hold exactly this chunk's query blocks")
    hm = _head_mask(head_mask, H)
    ws = _workspace(C.LCSR_WS_BLOCK_ATTN, prob, 0, 0, q.device, workspace)
    _check(C.load().lcsr_block_sparse_attn_prefill(
        ctypes.byref(prob), idx.data_ptr(), cnt.data_ptr(), pattern.max_blocks, _ptr(hm),
        out.data_ptr(), _dtype_code(out), out.stride(0), out.stride(1),
        _dense_rows(lse, H, n, "lse"), None if stats is None else stats.data_ptr(), ws.data_ptr(),
        ws.numel(), _stream(stream)))
    return out, lse


def block_sparse_recall_check(q, k_cache, chunk_start, rope, dca, sm_scale, pattern, rows,
                              head_mask=None, stream=None):
    """(lse_full, lse_sparse, recall), each [H, n_rows], of a block-sparse
    pattern (lcsr_block_sparse_recall_check)."""
    prob = _problem(q, k_cache, None, chunk_start, rope, dca, sm_scale)
    H, n = q.shape[0], rows.numel()
    n_qb = -(-q.shape[1] // 64)
    if rows.dtype != torch.int32 or not rows.is_contiguous():
        raise TypeError("rows must be a contiguous int32 tensor")
    idx, cnt = pattern.idx[:, :n_qb], pattern.cnt[:, :n_qb]
    if not (idx.is_contiguous() and cnt.is_contiguous()):
        raise ValueError("pattern buffers must hold exactly this chunk's query blocks")
    outs = [torch.empty((H, n), dtype=torch.float32, device=q.device) for _ in range(3)]
    hm = _head_mask(head_mask, H)
    _check(C.load().lcsr_block_sparse_recall_check(
        ctypes.byref(prob), idx.data_ptr(), cnt.data_ptr(), pattern.max_blocks, _ptr(hm),
        rows.data_ptr(), n, outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
        _stream(stream)))
    return tuple(outs)


def vs_pattern_estimate(q, k_cache, chunk_start, rope, dca, sm_scale, n_vert, n_slash,
                        pattern, last_q=64, head_mask=None, vert_score=None,
                        slash_score=None, select_only=False, workspace=None, stream=None):
    """Fill `pattern` with each head's verticals and slashes (lcsr_vs_pattern_estimate)."""
    prob = _problem(q, k_cache, None, chunk_start, rope, dca, sm_scale)
    H = q.shape[0]
    if len(n_vert) != H or len(n_slash) != H:
        raise ValueError("one budget per query head")
    nv = _host_i32(n_vert)
    ns = _host_i32(n_slash)
    hm = _head_mask(head_mask, H)
    ws = _workspace(C.LCSR_WS_ESTIMATE, prob, pattern.max_vert, pattern.max_slash, q.device,
                    workspace)
    pat = pattern.c()
    flags = C.LCSR_EST_SELECT_ONLY if select_only else 0
    _check(C.load().lcsr_vs_pattern_estimate(
        ctypes.byref(prob), int(last_q), _ptr(nv), _ptr(ns), _ptr(hm), ctypes.byref(pat),
        None if vert_score is None else vert_score.data_ptr(),
        None if slash_score is None else slash_score.data_ptr(), flags, ws.data_ptr(),
        ws.numel(), _stream(stream)))
    return pattern


def vs_sparse_attn_prefill(q, k_cache, v_cache, chunk_start, rope, dca, sm_scale, pattern,
                           out=None, out_dtype=torch.float32, lse=None, stats=None,
                           head_mask=None, dense=False, workspace=None, stream=None):
    """Sparse causal attention of the chunk's rows (lcsr_vs_sparse_attn_prefill).

    Returns (out [H, L, D], lse [H, L] or None)."""
    prob = _problem(q, k_cache, v_cache, chunk_start, rope, dca, sm_scale)
    H, L, D = q.shape
    if out is None:
        out = torch.empty((H, L, D), dtype=out_dtype, device=q.device)
    ms = 1 if pattern is None else pattern.max_slash
    mv = 1 if pattern is None else pattern.max_vert
    ws = _workspace(C.LCSR_WS_ATTN, prob, mv, ms, q.device, workspace)
    pat_s = None if pattern is None else pattern.c()
    pat = None if pat_s is None else ctypes.byref(pat_s)
    hm = _head_mask(head_mask, H)
    _check(C.load().lcsr_vs_sparse_attn_prefill(
        ctypes.byref(prob), pat, _ptr(hm), out.data_ptr(), _dtype_code(out),
        out.stride(0), out.stride(1), _dense_rows(lse, q.shape[0], q.shape[1], "lse"),
        None if stats is None else stats.data_ptr(), C.LCSR_ATTN_DENSE if dense else 0,
        ws.data_ptr(), ws.numel(), _stream(stream)))
    return out, lse


def attn_decode(q, k_cache, v_cache, row_start, rope, dca, sm_scale, out=None,
                out_dtype=torch.float32, lse=None, workspace=None, stream=None):
    """Decode-step attention of the newest rows (lcsr_attn_decode): q [H, n, D]
    holds tokens row_start .. row_start + n - 1, whose K/V are in the caches;
    every key up to each row, DCA logits.  Returns (out [H, n, D], lse or None)."""
    prob = _problem(q, k_cache, v_cache, row_start, rope, dca, sm_scale)
    H, n, D = q.shape
    if out is None:
        out = torch.empty((H, n, D), dtype=out_dtype, device=q.device)
    ws = _workspace(C.LCSR_WS_DECODE, prob, 0, 0, q.device, workspace)
    _check(C.load().lcsr_attn_decode(
        ctypes.byref(prob), out.data_ptr(), _dtype_code(out), out.stride(0), out.stride(1),
        _dense_rows(lse, H, n, "lse"), ws.data_ptr(), ws.numel(), _stream(stream)))
    return out, lse


def attn_decode_noalloc(q, k_cache, v_cache, row_start, rope, dca, sm_scale, out, lse=None,
                        stream=None):
    """attn_decode on the library's static scratch (lcsr_attn_decode_noalloc):
    no workspace and no allocation, so `out` (and `lse`, if wanted) must be
    given.  Calls that may overlap on one GPU must not use it concurrently."""
    prob = _problem(q, k_cache, v_cache, row_start, rope, dca, sm_scale)
    H, n, D = q.shape
    _check(C.load().lcsr_attn_decode_noalloc(
        ctypes.byref(prob), out.data_ptr(), _dtype_code(out), out.stride(0), out.stride(1),
        _dense_rows(lse, H, n, "lse"), _stream(stream)))
    return out, lse


def attn_recall_check(q, k_cache, chunk_start, rope, dca, sm_scale, pattern, rows,
                      head_mask=None, workspace=None, stream=None):
    """(lse_full, lse_sparse, recall), each [H, n_rows] (lcsr_attn_recall_check)."""
    prob = _problem(q, k_cache, None, chunk_start, rope, dca, sm_scale)
    H = q.shape[0]
    n = rows.numel()
    outs = [torch.empty((H, n), dtype=torch.float32, device=q.device) for _ in range(3)]
    ws = _workspace(C.LCSR_WS_RECALL, prob, pattern.max_vert, pattern.max_slash, q.device,
                    workspace)
    pat = pattern.c()
    hm = _head_mask(head_mask, H)
    if rows.dtype != torch.int32 or not rows.is_contiguous():
        raise TypeError("rows must be a contiguous int32 tensor")
    _check(C.load().lcsr_attn_recall_check(
        ctypes.byref(prob), ctypes.byref(pat), _ptr(hm), rows.data_ptr(), n,
        outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), ws.data_ptr(), ws.numel(),
        _stream(stream)))
    return tuple(outs)
