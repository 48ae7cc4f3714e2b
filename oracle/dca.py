"""Dual Chunk Attention position maps (integer arithmetic).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[Qwen2.5-1M explainer] Length Extrapolation describes three attention
patterns qualitatively: pairs in the same chunk keep their original relative
position (intra); pairs in non-adjacent chunks are remapped as a repeated
sequence so that no distance exceeds the training length (inter); adjacent
chunks keep continuity, with original positions inside a local window and
the inter rule elsewhere (successive).

Reading (the pages give no formulas): with C the largest position + 1 (the
training length, 262,144 for Qwen2.5-1M) and W the local window, keys repeat
with period S = C - W:
    key position           P_k(j)       = j mod S
    intra query position   P_intra(i)   = i mod S
    succ  query position   P_succ(i)    = S + (i mod S) if (i mod S) < W else C - 1
    inter query position   P_inter(i)   = C - 1
and the pair (i, j) uses intra / succ / inter when floor(i/S) - floor(j/S) is
0 / 1 / >= 2.  Every relative position then lies in [0, C-1]; intra pairs and
successive pairs with (i mod S) < W get exactly i - j.  chunk == 0 turns DCA
off (all positions are the token index).
"""

import numpy as np


def _period(chunk, local):
    if chunk <= 0:
        return None
    if not 0 <= local < chunk:
        raise ValueError("need 0 <= local < chunk")
    return chunk - local


def dca_position_maps(tok, chunk, local):
    """Per-token positions {pk, intra, succ, inter} (int64 arrays)."""
    tok = np.asarray(tok, dtype=np.int64)
    period = _period(chunk, local)
    if period is None:
        return {"pk": tok.copy(), "intra": tok.copy(), "succ": tok.copy(),
                "inter": tok.copy()}
    ip = tok % period
    succ = np.where(ip < local, period + ip, chunk - 1)
    return {"pk": ip, "intra": ip.copy(), "succ": succ.astype(np.int64),
            "inter": np.full_like(tok, chunk - 1)}


def dca_chunk_of(tok, chunk, local):
    """Index of the DCA chunk holding each token (0 when DCA is off)."""
    tok = np.asarray(tok, dtype=np.int64)
    period = _period(chunk, local)
    if period is None:
        return np.zeros_like(tok)
    return tok // period


def query_positions(i, js, chunk, local):
    """Position at which query row i is rotated when it attends each key js."""
    js = np.asarray(js, dtype=np.int64)
    period = _period(chunk, local)
    if period is None:
        return np.full_like(js, int(i))
    maps = dca_position_maps(np.array([i]), chunk, local)
    rel = int(i) // period - js // period
    return np.where(rel == 0, maps["intra"][0],
                    np.where(rel == 1, maps["succ"][0], maps["inter"][0]))


def relative_positions(i, js, chunk, local):
    """P_q(i, j) - P_k(j): the relative position RoPE sees for each pair."""
    js = np.asarray(js, dtype=np.int64)
    pk = dca_position_maps(js, chunk, local)["pk"]
    return query_positions(i, js, chunk, local) - pk
