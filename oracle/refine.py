"""Sparsity refinement step (budget update), integer control logic.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[Qwen2.5-1M explainer] Chunked Prefill / Sparsity Refinement: heads whose
attention recall falls under a threshold get a larger vertical and slash
budget.  Reading (the page does not give the increment): threshold 0.9 on
the head's mean recall over the sampled rows; both budgets double, capped at
the number of keys; at most three rounds.

Heads with a fixed pattern kind grow their own size (same reading: double,
capped): a block-sparse head its kept blocks per query block (cap: the key
blocks of the context), an A-shape head its recent window (cap: the number of
keys; the sink count stays).
"""

import numpy as np


def refine_budgets(recall_mean, n_vert, n_slash, n_keys, threshold=0.9):
    """New (n_vert, n_slash, raised) for one refinement round.

    recall_mean: [H] head means; heads below the threshold whose budgets can
    still grow are raised; `raised` is the boolean mask of those heads.
    """
    recall_mean = np.asarray(recall_mean, dtype=np.float64)
    n_vert = np.asarray(n_vert, dtype=np.int64).copy()
    n_slash = np.asarray(n_slash, dtype=np.int64).copy()
    low = recall_mean < threshold
    can_grow = (n_vert < n_keys) | (n_slash < n_keys)
    raised = low & can_grow
    n_vert[raised] = np.minimum(2 * n_vert[raised], n_keys)
    n_slash[raised] = np.minimum(2 * n_slash[raised], n_keys)
    return n_vert, n_slash, raised


def refine_sizes(recall_mean, kinds, sizes, n_keys, threshold=0.9):
    """One refinement round over heads of any kind.

    kinds[h] in {"vs", "block", "a_shape"}; sizes[h] is (n_vert, n_slash),
    (n_blocks,) or (n_sink, n_local).  Returns (new sizes, raised mask)."""
    n_kb = -(-int(n_keys) // 64)
    new, raised = [], []
    for h, kind in enumerate(kinds):
        low = float(recall_mean[h]) < threshold
        sz = tuple(int(x) for x in sizes[h])
        if kind == "vs":
            grow = low and (sz[0] < n_keys or sz[1] < n_keys)
            nxt = (min(2 * sz[0], n_keys), min(2 * sz[1], n_keys)) if grow else sz
        elif kind == "block":
            grow = low and sz[0] < n_kb
            nxt = (min(2 * sz[0], n_kb),) if grow else sz
        elif kind == "a_shape":
            grow = low and sz[1] < n_keys
            nxt = (sz[0], min(2 * sz[1], n_keys)) if grow else sz
        else:
            raise ValueError(kind)
        new.append(nxt)
        raised.append(grow)
    return new, np.array(raised, dtype=bool)
