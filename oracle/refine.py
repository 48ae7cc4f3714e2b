"""Sparsity refinement step (budget update), integer control logic.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[Qwen2.5-1M explainer] Chunked Prefill / Sparsity Refinement: heads whose
attention recall falls under a threshold get a larger vertical and slash
budget.  Reading (the page does not give the increment): threshold 0.9 on
the head's mean recall over the sampled rows; both budgets double, capped at
the number of keys; at most three rounds.
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
