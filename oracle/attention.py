"""Dense and vertical-slash sparse attention rows, and attention recall (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Rows are computed one at a time, exactly as defined: logits over a key set,
a softmax over that set, the weighted sum of values and the natural-log
logsumexp.  Grouped-query attention: query head h reads KV head
h // (H / H_kv) ([architecture overview] §4.6 repeat_interleave mapping); the
caller passes the KeyContext of that KV head.
"""

import numpy as np

from .dca import dca_position_maps, query_positions
from .rope import bf16_round64, fp16_round64, rope_rotate


class KeyContext:
    """Pre-RoPE keys and the values of one KV head, plus the RoPE setup.

    K and V are [N, D].  Rotated keys are computed once per context and
    cached: at DCA key positions (attention) and at the plain token index
    (the continuous positions used for pattern selection).

    operands="fp64" (the parity reference) keeps rotated keys and queries
    exact.  operands="bf16" or "fp16" models a matrix-core operand type: the
    rotated keys (the K cache, stored once at the DCA key position:
    [Qwen2.5-1M explainer] 推論フレームワーク) and the rotated queries enter
    the QK^T products rounded to the nearest (ties to even) value of that
    type from their exact fp64 rotation.  Every other step stays fp64.
    These modes only separate the operand rounding from the rest of an
    error; nothing is asserted against them.
    """

    _ROUND = {"bf16": bf16_round64, "fp16": fp16_round64}

    def __init__(self, K, V, inv_freq, dca_chunk=0, dca_local=0, operands="fp64"):
        if operands not in ("fp64", "bf16", "fp16"):
            raise ValueError("operands must be 'fp64', 'bf16' or 'fp16'")
        self.operands = operands
        self.K = np.asarray(K, dtype=np.float64)
        self.V = None if V is None else np.asarray(V, dtype=np.float64)
        self.inv_freq = np.asarray(inv_freq, dtype=np.float64)
        self.dca_chunk = int(dca_chunk)
        self.dca_local = int(dca_local)
        self._k_dca = None
        self._k_cont = None

    def operand(self, x):
        """A rotated vector as it enters a QK^T product."""
        return x if self.operands == "fp64" else self._ROUND[self.operands](x)

    @property
    def n_keys(self):
        return self.K.shape[0]

    def _pk(self):
        return dca_position_maps(np.arange(self.n_keys), self.dca_chunk,
                                 self.dca_local)["pk"]

    def k_dca(self):
        """Keys rotated at the DCA key position P_k(j), as the cache holds them."""
        if self._k_dca is None:
            k = rope_rotate(self.K, self._pk(), self.inv_freq)
            self._k_dca = self.operand(k)
        return self._k_dca

    def k_cont(self):
        """Keys rotated at their own index j (continuous positions).

        From a rounded cache, the cached key turns on by j - P_k(j), a
        multiple of the key period: R(j) k = R(j - P_k(j)) R(P_k(j)) k."""
        if self._k_cont is None:
            idx = np.arange(self.n_keys)
            if self.operands != "fp64":
                self._k_cont = rope_rotate(self.k_dca(), idx - self._pk(), self.inv_freq)
            else:
                self._k_cont = rope_rotate(self.K, idx, self.inv_freq)
        return self._k_cont


def attention_logits(q_row, i, ctx, js, sm_scale):
    """l_ij = sm_scale * <R(P_q(i, j)) q_i, R(P_k(j)) k_j> for keys js.

    DCA positions ([Qwen2.5-1M explainer] アルゴリズム: attention weights are
    computed with the non-continuous DCA relative positions); sm_scale is
    the YaRN temperature 1/(t sqrt(D)).
    """
    js = np.asarray(js, dtype=np.int64)
    out = np.empty(js.shape[0], dtype=np.float64)
    if js.size == 0:
        return out
    pq = query_positions(i, js, ctx.dca_chunk, ctx.dca_local)
    keys = ctx.k_dca()
    for p in np.unique(pq):
        sel = pq == p
        q_rot = ctx.operand(rope_rotate(np.asarray(q_row, np.float64), p, ctx.inv_freq))
        out[sel] = keys[js[sel]] @ q_rot
    return sm_scale * out


def _softmax_row(logits, values):
    """(o, lse) of softmax(logits) @ values; an empty set gives (0, -inf)."""
    if logits.size == 0:
        return np.zeros(values.shape[1]), -np.inf
    m = np.max(logits)
    e = np.exp(logits - m)
    z = np.sum(e)
    return (e / z) @ values, m + np.log(z)


def dense_causal_rows(q_rows, rows, ctx, sm_scale):
    """Causal attention of query rows over every key j <= i (DCA logits)."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, ctx.V.shape[1]))
    lse = np.zeros(rows.size)
    for a, i in enumerate(rows):
        js = np.arange(i + 1)
        lg = attention_logits(q_rows[a], i, ctx, js, sm_scale)
        out[a], lse[a] = _softmax_row(lg, ctx.V[js])
    return out, lse


def critical_set(i, verts, slashes):
    """C_i = {v in verts : v <= i} U {i - o : o in slashes, o <= i}, as a
    sorted set (each key once).

    [Qwen2.5-1M explainer] 疎アテンション: attention is computed over the
    critical tokens chosen by the vertical (key column) and slash (diagonal
    offset i - j) patterns; Chunked Prefill defines recall over the set C.
    """
    verts = np.asarray(verts, dtype=np.int64)
    slashes = np.asarray(slashes, dtype=np.int64)
    a = verts[verts <= i]
    b = i - slashes[slashes <= i]
    return np.union1d(a, b)


def sparse_rows(q_rows, rows, ctx, verts, slashes, sm_scale):
    """Vertical-slash sparse attention of query rows.

    Returns (out [n, D], lse [n], set sizes [n]).
    """
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, ctx.V.shape[1]))
    lse = np.zeros(rows.size)
    sizes = np.zeros(rows.size, dtype=np.int64)
    for a, i in enumerate(rows):
        js = critical_set(i, verts, slashes)
        sizes[a] = js.size
        lg = attention_logits(q_rows[a], i, ctx, js, sm_scale)
        out[a], lse[a] = _softmax_row(lg, ctx.V[js])
    return out, lse, sizes


def _lse(logits):
    if logits.size == 0:
        return -np.inf
    m = np.max(logits)
    return m + np.log(np.sum(np.exp(logits - m)))


def attention_recall(q_rows, rows, ctx, verts, slashes, sm_scale):
    """Attention recall per row ([Qwen2.5-1M explainer] Chunked Prefill):
    lse_full over all j <= i, lse_sparse over C_i, recall =
    exp(lse_sparse - lse_full).

    Reading: both sums use the logits the attention actually computes (DCA
    positions, YaRN temperature); the page writes q^T k / sqrt(D), which is
    the special case without DCA and with s = 1.
    """
    rows = np.asarray(rows, dtype=np.int64)
    full = np.zeros(rows.size)
    sparse = np.zeros(rows.size)
    for a, i in enumerate(rows):
        lg = attention_logits(q_rows[a], i, ctx, np.arange(i + 1), sm_scale)
        full[a] = _lse(lg)
        cs = critical_set(i, verts, slashes)
        sparse[a] = _lse(lg[cs])
    return full, sparse, np.exp(sparse - full)
