"""Block-sparse head pattern: block scores from pooled queries and keys,
per-query-block selection, attention inside the chosen key blocks (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[architecture overview] §4.2 lists, beside the vertical and slash patterns,
a block pattern among the stable head patterns MInference observes; §4.3
describes selectors that score whole KV blocks for each query and attend
only inside the high-scoring blocks.  [Qwen2.5-1M explainer] アルゴリズム:
selection uses continuous relative positions, attention the DCA positions.

Readings (the pages name the pattern but give no procedure):
* blocks hold 64 queries or 64 keys, aligned to the token index (block b is
  tokens 64 b .. 64 b + 63; the chunk starts on a block edge);
* the score of (query block, key block) is sm_scale times the inner product
  of the block means of R(i) q_i and R(j) k_j (continuous positions, as for
  the vertical-slash estimate); by bilinearity it is the mean of the
  continuous-position logits over the block pair;
* each query block keeps its diagonal key block (the one holding its first
  query) and the k - 1 best earlier key blocks, ranked by (score desc, index
  asc), k = min(budget, diag + 1); the list is ascending;
* row i attends to every key j <= i inside a kept block, with DCA logits.
"""

import numpy as np

from .attention import attention_logits, _softmax_row
from .estimate import select_top
from .rope import rope_rotate

BLOCK = 64


def block_scores(q_chunk, chunk_start, ctx, sm_scale):
    """Scores [n_qb, n_kb] of one head's chunk: query blocks of the chunk
    against key blocks [0, n_kb) of the keys up to the chunk's end; -inf
    above the diagonal."""
    q_chunk = np.asarray(q_chunk, np.float64)
    n = q_chunk.shape[0]
    c1 = chunk_start + n
    n_qb = -(-n // BLOCK)
    n_kb = -(-c1 // BLOCK)
    rows = np.arange(chunk_start, c1)
    q_cont = rope_rotate(q_chunk, rows, ctx.inv_freq)
    k_cont = ctx.k_cont()[:c1]
    qm = np.stack([q_cont[b * BLOCK:(b + 1) * BLOCK].mean(axis=0) for b in range(n_qb)])
    km = np.stack([k_cont[b * BLOCK:(b + 1) * BLOCK].mean(axis=0) for b in range(n_kb)])
    s = sm_scale * (qm @ km.T)
    diag = chunk_start // BLOCK + np.arange(n_qb)
    s[np.arange(n_kb)[None, :] > diag[:, None]] = -np.inf
    return s


def select_blocks(scores_row, diag, k):
    """Kept key blocks of one query block, ascending: the diagonal block and
    the k - 1 best of blocks 0 .. diag - 1 (ties to the lower index)."""
    k = max(1, min(int(k), diag + 1))
    earlier = select_top(np.asarray(scores_row)[:diag], k - 1)
    return np.sort(np.append(earlier, diag)).astype(np.int64)


def block_key_set(i, blocks):
    """Keys of row i: every j <= i inside the kept blocks, sorted."""
    js = [np.arange(b * BLOCK, min((b + 1) * BLOCK, i + 1)) for b in np.sort(blocks)]
    js = [x for x in js if x.size]
    return np.concatenate(js) if js else np.zeros(0, dtype=np.int64)


def block_sparse_rows(q_rows, rows, ctx, blocks_of_row, sm_scale):
    """Attention of query rows over their kept key blocks.

    blocks_of_row(i) -> kept key blocks of row i.  Returns (out [n, D],
    lse [n], set sizes [n])."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, ctx.V.shape[1]))
    lse = np.zeros(rows.size)
    sizes = np.zeros(rows.size, dtype=np.int64)
    for a, i in enumerate(rows):
        js = block_key_set(int(i), blocks_of_row(int(i)))
        sizes[a] = js.size
        lg = attention_logits(q_rows[a], int(i), ctx, js, sm_scale)
        out[a], lse[a] = _softmax_row(lg, ctx.V[js])
    return out, lse, sizes
