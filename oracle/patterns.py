"""Fixed sparse patterns and the per-head pattern search.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* [architecture overview] §4.1 (sliding window and StreamingLLM's attention
  sink): a row keeps the first few tokens of the sequence (the sinks) and its
  most recent W tokens.  MInference calls this head pattern "A-shape".
* [architecture overview] §4.2: almost every head falls into one of a few
  stable patterns, so sparsification gives each head one pattern and a span.
* [Qwen2.5-1M explainer] 疎アテンション: an offline search fixes each head's
  configuration (its numbers of verticals and slashes) before inference;
  Chunked Prefill: attention recall measures how much of the full softmax
  mass a sparse set keeps.

Readings (the pages name the search but give no procedure):
  - a candidate is a pattern kind with its sizes: vertical-slash budgets
    (n_vert, n_slash) chosen by the estimate, or an A-shape (n_sink, n_local);
  - a head's score for a candidate is its attention recall averaged over the
    sampled rows of every calibration chunk;
  - each head takes the candidate with the highest score; on an exact tie the
    earlier candidate in the caller's list wins (callers list cheaper ones
    first).
"""

import numpy as np


def a_shape_set(i, n_sink, n_local):
    """Keys row i attends to under an A-shape head: j <= i with j < n_sink
    (an attention sink) or i - j < n_local (the recent window), sorted."""
    js = np.arange(i + 1, dtype=np.int64)
    keep = (js < n_sink) | (i - js < n_local)
    return js[keep]


def a_shape_lists(n_sink, n_local, n_keys):
    """The A-shape as vertical and slash lists over n_keys keys: verticals
    0 .. n_sink - 1 (the sink columns) and slash offsets 0 .. n_local - 1
    (the window's diagonals), each cut at n_keys."""
    return (np.arange(min(n_sink, n_keys), dtype=np.int64),
            np.arange(min(n_local, n_keys), dtype=np.int64))


def choose_candidates(scores):
    """scores [n_candidates, H] (mean recall per candidate and head) ->
    int [H]: per head the candidate with the highest score, the earliest one
    on an exact tie."""
    scores = np.asarray(scores, dtype=np.float64)
    n_c, n_h = scores.shape
    best = np.zeros(n_h, dtype=np.int64)
    for h in range(n_h):
        for c in range(1, n_c):
            if scores[c, h] > scores[best[h], h]:
                best[h] = c
    return best
