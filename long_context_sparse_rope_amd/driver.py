"""Chunked sparse prefill of one attention layer, with sparsity refinement.

The loop of the page "論文解説: Qwen2.5-1M" (0h-n0.github.io), section
"アルゴリズム: DCAと疎アテンションの統合": the prompt is processed in prefill
chunks; for each chunk the critical tokens are chosen from the chunk's last
queries with continuous positions, then the chunk's attention is computed
over them with DCA positions.  Chunked Prefill gives the 32,768-token chunk
and the attention-recall check used by the refinement.

Heads may also carry a fixed A-shape pattern (attention sinks plus a recent
window, the page deepseekmodel.com long-context architecture overview, §4.1)
or a block-sparse one (whole 64-key blocks chosen per 64-query block, §4.2 and
§4.3 there) instead of an estimated vertical-slash one; §4.2 gives each head
one pattern.  `search_head_patterns` is the offline per-head search of the
0h-n0.github.io page, section 疎アテンション, scored by attention recall
(section Chunked Prefill).

Every numeric step runs in liblcsr.so; this module only sequences the calls
on one stream and owns the KV cache buffers.
"""

import math

import numpy as np
import torch

from . import ops


def _head_means(recall):
    """Mean recall of each head over its sampled rows, formed on the host
    from the copied fp32 recalls (exactly rounded sums, so the order of the
    rows does not matter)."""
    r = recall.cpu().numpy().astype(np.float64)
    return np.array([math.fsum(row) / row.size for row in r])


class ChunkedSparsePrefill:
    """One layer's KV cache plus the calls of the chunk loop.

    The K cache is fp16 and the V cache bf16, both [H_kv, max_ctx, D]; keys
    are stored rotated at their DCA key position (fp16: the QK^T operand
    type of the kernels).  Budgets are per query head and may be raised by
    `refine_chunk`.  A head is a vertical-slash head (budgets n_vert,
    n_slash, pattern from the estimate), an A-shape head (n_sink, n_local, no
    estimate) or a block-sparse head (n_blocks key blocks per query block);
    see `set_head_patterns`.
    """

    def __init__(self, n_heads, n_kv_heads, head_dim, max_ctx, rope, dca, sm_scale,
                 n_vert, n_slash, last_q=64, device="cuda", max_vert=None, max_slash=None):
        self.H, self.Hkv, self.D = n_heads, n_kv_heads, head_dim
        self.max_ctx = int(max_ctx)
        self.rope, self.dca, self.sm_scale = rope, dca, float(sm_scale)
        self.last_q = last_q
        self.device = torch.device(device)
        self.n_vert = [int(n_vert)] * n_heads if isinstance(n_vert, int) else list(n_vert)
        self.n_slash = [int(n_slash)] * n_heads if isinstance(n_slash, int) else list(n_slash)
        self.a_shape = [None] * n_heads      # (n_sink, n_local) of A-shape heads
        self.blocks = [None] * n_heads       # n_blocks of block-sparse heads
        self.block_pattern = None
        self.k_cache = torch.empty((n_kv_heads, self.max_ctx, head_dim), dtype=torch.float16,
                                   device=self.device)
        self.v_cache = torch.empty((n_kv_heads, self.max_ctx, head_dim), dtype=torch.bfloat16,
                                   device=self.device)
        mv = max_vert or max(self.n_vert)
        ms = max_slash or max(self.n_slash)
        self.pattern = ops.Pattern(n_heads, mv, ms, self.device)

    def append_kv(self, k_chunk, v_chunk, chunk_start):
        """Rotate the chunk's keys into the K cache at P_k and copy V."""
        n = k_chunk.shape[1]
        pos = ops.dca_positions(chunk_start, n, self.dca, self.device)["pk"]
        ops.rope_yarn_apply(k_chunk, pos, self.rope,
                            out=self.k_cache[:, chunk_start:chunk_start + n])
        ops.rope_yarn_apply(v_chunk, None, self.rope, rotate=False,
                            out=self.v_cache[:, chunk_start:chunk_start + n])

    def set_head_patterns(self, configs):
        """One configuration per query head: {"kind": "vs", "n_vert": a,
        "n_slash": b}, {"kind": "a_shape", "n_sink": s, "n_local": w} or
        {"kind": "block", "n_blocks": k}.  The pattern buffers grow to fit."""
        if len(configs) != self.H:
            raise ValueError("one configuration per query head")
        for h, c in enumerate(configs):
            if c["kind"] == "vs":
                self.n_vert[h], self.n_slash[h] = int(c["n_vert"]), int(c["n_slash"])
                self.a_shape[h], self.blocks[h] = None, None
            elif c["kind"] == "a_shape":
                self.a_shape[h], self.blocks[h] = (int(c["n_sink"]), int(c["n_local"])), None
            elif c["kind"] == "block":
                self.a_shape[h], self.blocks[h] = None, int(c["n_blocks"])
            else:
                raise ValueError(f"unknown pattern kind {c['kind']!r}")
        mv = max(self.n_vert + [a[0] for a in self.a_shape if a])
        ms = max(self.n_slash + [a[1] for a in self.a_shape if a])
        if mv > self.pattern.max_vert or ms > self.pattern.max_slash:
            self.pattern = ops.Pattern(self.H, max(mv, self.pattern.max_vert),
                                       max(ms, self.pattern.max_slash), self.device)

    def estimate(self, q_chunk, chunk_start, head_mask=None):
        """The chunk's pattern: the estimate for vertical-slash heads, the
        A-shape rows for the others (only heads in head_mask, if given)."""
        c1 = chunk_start + q_chunk.shape[1]
        sel = [head_mask is None or bool(head_mask[h]) for h in range(self.H)]
        blk = [sel[h] and self.blocks[h] is not None for h in range(self.H)]
        vs = [sel[h] and self.a_shape[h] is None and not blk[h] for h in range(self.H)]
        if any(vs):
            ops.vs_pattern_estimate(
                q_chunk, self.k_cache[:, :c1], chunk_start, self.rope, self.dca, self.sm_scale,
                self.n_vert, self.n_slash, self.pattern, last_q=self.last_q,
                head_mask=None if all(vs) else vs)
        sizes = sorted({self.a_shape[h] for h in range(self.H) if sel[h] and self.a_shape[h]})
        for size in sizes:
            ops.pattern_fill_a_shape(self.pattern, size[0], size[1], c1,
                                     head_mask=[sel[h] and self.a_shape[h] == size
                                                for h in range(self.H)])
        if any(blk):
            n_qb = -(-q_chunk.shape[1] // 64)
            mb = max(b for b in self.blocks if b is not None)
            bp = self.block_pattern
            if bp is None or bp.idx.shape[1] != n_qb or bp.max_blocks < mb:
                self.block_pattern = ops.BlockPattern(self.H, n_qb, mb, self.device)
                if bp is not None and bp.idx.shape[1] == n_qb:
                    # rows of heads not estimated now keep their lists
                    self.block_pattern.idx[:, :, :bp.max_blocks] = bp.idx
                    self.block_pattern.cnt.copy_(bp.cnt)
            ops.block_sparse_estimate(
                q_chunk, self.k_cache[:, :c1], chunk_start, self.rope, self.dca, self.sm_scale,
                [b or 1 for b in self.blocks], self.block_pattern, head_mask=blk)
        return self.pattern

    def attend(self, q_chunk, chunk_start, out=None, lse=None, stats=None, head_mask=None,
               dense=False):
        """The chunk's attention: one call for the vertical-slash and A-shape
        heads, one for the block-sparse heads, each on its own heads."""
        c1 = chunk_start + q_chunk.shape[1]
        sel = [head_mask is None or bool(head_mask[h]) for h in range(self.H)]
        blk = [sel[h] and self.blocks[h] is not None and not dense for h in range(self.H)]
        rest = [sel[h] and not blk[h] for h in range(self.H)]
        if not any(blk):
            return ops.vs_sparse_attn_prefill(
                q_chunk, self.k_cache[:, :c1], self.v_cache[:, :c1], chunk_start, self.rope,
                self.dca, self.sm_scale, None if dense else self.pattern, out=out, lse=lse,
                stats=stats, head_mask=head_mask, dense=dense)
        if out is None:
            out = torch.empty((self.H, q_chunk.shape[1], self.D), dtype=torch.float32,
                              device=self.device)
        if any(rest):
            ops.vs_sparse_attn_prefill(
                q_chunk, self.k_cache[:, :c1], self.v_cache[:, :c1], chunk_start, self.rope,
                self.dca, self.sm_scale, self.pattern, out=out, lse=lse, stats=stats,
                head_mask=rest)
        ops.block_sparse_attn_prefill(
            q_chunk, self.k_cache[:, :c1], self.v_cache[:, :c1], chunk_start, self.rope,
            self.dca, self.sm_scale, self.block_pattern, out=out, lse=lse, stats=stats,
            head_mask=blk)
        return out, lse

    def recall(self, q_chunk, chunk_start, rows, head_mask=None):
        """(lse_full, lse_sparse, recall) [H, n_rows] of the sampled rows,
        each head on its own pattern kind."""
        c1 = chunk_start + q_chunk.shape[1]
        sel = [head_mask is None or bool(head_mask[h]) for h in range(self.H)]
        blk = [sel[h] and self.blocks[h] is not None for h in range(self.H)]
        rest = [sel[h] and not blk[h] for h in range(self.H)]
        if not any(blk):
            return ops.attn_recall_check(q_chunk, self.k_cache[:, :c1], chunk_start, self.rope,
                                         self.dca, self.sm_scale, self.pattern, rows,
                                         head_mask=head_mask)
        bf, bs, br = ops.block_sparse_recall_check(
            q_chunk, self.k_cache[:, :c1], chunk_start, self.rope, self.dca, self.sm_scale,
            self.block_pattern, rows, head_mask=blk)
        if not any(rest):
            return bf, bs, br
        lf, ls, rc = ops.attn_recall_check(q_chunk, self.k_cache[:, :c1], chunk_start,
                                           self.rope, self.dca, self.sm_scale, self.pattern,
                                           rows, head_mask=rest)
        hb = torch.tensor([h for h in range(self.H) if blk[h]], device=self.device)
        lf[hb], ls[hb], rc[hb] = bf[hb], bs[hb], br[hb]
        return lf, ls, rc

    def prefill_chunk(self, q_chunk, k_chunk, v_chunk, chunk_start, out=None, lse=None,
                      stats=None):
        """One chunk: KV append, pattern estimate, sparse attention."""
        self.append_kv(k_chunk, v_chunk, chunk_start)
        self.estimate(q_chunk, chunk_start)
        return self.attend(q_chunk, chunk_start, out=out, lse=lse, stats=stats)

    def refine_chunk(self, q_chunk, chunk_start, rows, out, lse=None, threshold=0.9,
                     max_rounds=3):
        """Sparsity refinement for one chunk: heads whose mean recall over
        `rows` is under the threshold grow, are re-estimated (or re-filled)
        and re-attended; at most `max_rounds` rounds.  A vertical-slash head
        doubles both budgets (capped at the number of keys), a block-sparse
        head its kept blocks (capped at the key blocks), an A-shape head its
        window (capped at the number of keys; the sinks stay).  Raised sizes
        carry over to later chunks.  Returns the per-round head recalls (host
        float64 arrays)."""
        c1 = chunk_start + q_chunk.shape[1]
        history = []
        for _ in range(max_rounds + 1):
            _, _, rec = self.recall(q_chunk, chunk_start, rows)
            mean = _head_means(rec)
            history.append(mean)
            n_kb = -(-c1 // 64)

            def can_grow(h):
                if self.blocks[h] is not None:
                    return self.blocks[h] < n_kb
                if self.a_shape[h] is not None:
                    return self.a_shape[h][1] < c1
                return self.n_vert[h] < c1 or self.n_slash[h] < c1

            low = [bool(mean[h] < threshold) and can_grow(h) for h in range(self.H)]
            if len(history) > max_rounds or not any(low):
                break
            for h in range(self.H):
                if not low[h]:
                    continue
                if self.blocks[h] is not None:
                    self.blocks[h] = min(2 * self.blocks[h], n_kb)
                elif self.a_shape[h] is not None:
                    s_, w_ = self.a_shape[h]
                    self.a_shape[h] = (s_, min(2 * w_, c1))
                else:
                    self.n_vert[h] = min(2 * self.n_vert[h], c1)
                    self.n_slash[h] = min(2 * self.n_slash[h], c1)
            need_v = max([self.n_vert[h] for h in range(self.H)] +
                         [a[0] for a in self.a_shape if a])
            need_s = max([self.n_slash[h] for h in range(self.H)] +
                         [a[1] for a in self.a_shape if a])
            if need_v > self.pattern.max_vert or need_s > self.pattern.max_slash:
                old = self.pattern
                self.pattern = ops.Pattern(self.H, max(need_v, old.max_vert),
                                           max(need_s, old.max_slash), self.device)
                # keep the heads that are not re-estimated
                for h in range(self.H):
                    if not low[h]:
                        self.pattern.vert_idx[h, :old.max_vert] = old.vert_idx[h]
                        self.pattern.slash_idx[h, :old.max_slash] = old.slash_idx[h]
                        self.pattern.vert_cnt[h] = old.vert_cnt[h]
                        self.pattern.slash_cnt[h] = old.slash_cnt[h]
            self.estimate(q_chunk, chunk_start, head_mask=low)
            self.attend(q_chunk, chunk_start, out=out, lse=lse, head_mask=low)
        return history

    def run(self, q, k, v, chunk_size, out=None, lse=None, stats=None):
        """Whole-prompt chunked prefill; q [H, N, D], k/v [H_kv, N, D]."""
        N = q.shape[1]
        if out is None:
            out = torch.empty((self.H, N, self.D), dtype=torch.float32, device=self.device)
        # the library writes lse as a dense [H, rows] block per call
        part = None if lse is None else torch.empty((self.H, min(chunk_size, N)),
                                                    dtype=torch.float32, device=self.device)
        for c0 in range(0, N, chunk_size):
            c1 = min(N, c0 + chunk_size)
            lc = None if part is None else part[:, :c1 - c0]
            if lc is not None and c1 - c0 < part.shape[1]:
                lc = lc.contiguous()
            self.prefill_chunk(q[:, c0:c1], k[:, c0:c1], v[:, c0:c1], c0,
                               out=out[:, c0:c1], lse=lc, stats=stats)
            if lse is not None:
                lse[:, c0:c1].copy_(lc)
        return out


def search_head_patterns(layer, q, chunks, candidates, rows):
    """Offline per-head pattern search over a calibration prompt.

    The layer's KV cache must already hold the prompt (append_kv for every
    chunk).  For each candidate (a configuration as in set_head_patterns)
    every head takes that candidate, each calibration chunk (c0, length) of
    `chunks` gets its pattern (estimate or A-shape fill) and the attention
    recall of its `rows` (row offsets within the chunk: one int32 device
    tensor, or one per chunk); a head's score is its recall averaged over the
    rows of a chunk, then over the chunks.  Each head takes the candidate
    with the highest score, the earlier one on an exact tie.  The layer's own
    configuration is restored afterwards.

    Returns (choice: list of H candidate indices, scores: float64 array
    [n_candidates, H]).
    """
    saved = (list(layer.n_vert), list(layer.n_slash), list(layer.a_shape), list(layer.blocks))
    H = layer.H
    scores = np.zeros((len(candidates), H))
    try:
        for ci, cand in enumerate(candidates):
            layer.set_head_patterns([cand] * H)
            for k, (c0, n) in enumerate(chunks):
                r = rows[k] if isinstance(rows, (list, tuple)) else rows
                layer.estimate(q[:, c0:c0 + n], c0)
                _, _, rec = layer.recall(q[:, c0:c0 + n], c0, r)
                scores[ci] += _head_means(rec)
            scores[ci] /= len(chunks)
    finally:
        layer.n_vert, layer.n_slash, layer.a_shape, layer.blocks = saved
    choice = []
    for h in range(H):
        best = 0
        for c in range(1, len(candidates)):
            if scores[c, h] > scores[best, h]:
                best = c
        choice.append(best)
    return choice, scores
