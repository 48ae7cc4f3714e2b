"""Vertical-slash pattern estimate and top-k selection (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[Qwen2.5-1M explainer] 疎アテンション: at inference time the attention
between the last queries (last_q) and all keys is computed, and critical
tokens are chosen dynamically along vertical lines (key columns) and slash
lines (diagonals).  Chunked Prefill: the last 64 tokens *of each chunk* are
used.  アルゴリズム: selection uses continuous relative positions, so the
slash lines stay straight.

Readings (the pages give no formulas):
* scores are row-softmax probabilities A of the estimate rows, with the same
  temperature as the attention and continuous positions (R(i) q_i,
  R(j) k_j); keys are [0, chunk_end) with j <= r (no future keys exist in
  chunked prefill);
* vertical score v_j = sum_r A[r, j]; slash score s_o = sum_r A[r, r - o];
* the estimate rows are the last min(last_q, chunk_len) rows of the chunk;
* selection keeps the min(k, n) largest scores, ordered by (score desc,
  index asc), and returns them in ascending index order.
"""

import numpy as np

from .rope import rope_rotate


def estimate_rows(chunk_start, chunk_len, last_q=64):
    """Absolute row indices of the estimate queries of one prefill chunk."""
    c1 = chunk_start + chunk_len
    return np.arange(max(chunk_start, c1 - last_q), c1, dtype=np.int64)


def estimate_scores(q_rows, rows, ctx, n_keys, sm_scale):
    """(v, s): vertical scores over keys [0, n_keys) and slash scores over
    offsets [0, n_keys) for one query head."""
    rows = np.asarray(rows, dtype=np.int64)
    q_rot = ctx.operand(rope_rotate(np.asarray(q_rows, np.float64), rows, ctx.inv_freq))
    keys = ctx.k_cont()[:n_keys]
    logits = sm_scale * (q_rot @ keys.T)
    logits[rows[:, None] < np.arange(n_keys)[None, :]] = -np.inf
    logits -= np.max(logits, axis=1, keepdims=True)
    probs = np.exp(logits)
    probs /= np.sum(probs, axis=1, keepdims=True)
    v = np.sum(probs, axis=0)
    s = np.zeros(n_keys)
    for a, r in enumerate(rows):
        s[: r + 1] += probs[a, r::-1]      # offset o = r - j, j = r .. 0
    return v, s


def select_top(scores, k):
    """Indices of the min(k, n) largest scores; ties go to the lower index;
    returned in ascending order (int64)."""
    scores = np.asarray(scores)
    n = scores.shape[0]
    k = max(0, min(int(k), n))
    order = np.lexsort((np.arange(n), -scores.astype(np.float64)))
    return np.sort(order[:k]).astype(np.int64)


def select_pattern(v, s, n_vert, n_slash):
    """(vertical key columns, slash offsets) chosen from one head's scores."""
    return select_top(v, n_vert), select_top(s, n_slash)
