"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs."""

import math

import numpy as np
import torch

import oracle
import long_context_sparse_rope_amd as L

DEV = "cuda"

# Output bar for bf16 inputs with fp32 accumulation, against the fp64 oracle
# with exact rotated operands.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def rope_of(cfg, blend=False):
    return L.RopeConfig(base=cfg.rope_base, yarn_factor=cfg.yarn_factor,
                        orig_max_pos=cfg.yarn_orig_max_pos, freq_blend=blend)


def dca_of(cfg):
    return L.DcaConfig(cfg.dca_chunk, cfg.dca_local)


def product_sm(cfg):
    """The logit scale as the library forms it (lcsr_softmax_scale), checked
    against the oracle's fp64 YaRN temperature to float rounding."""
    sm = L.softmax_scale(cfg.head_dim, rope_of(cfg))
    ref = oracle.softmax_scale(cfg.head_dim, cfg.yarn_factor)
    assert abs(sm - ref) <= 2 ** -23 * ref, (sm, ref)
    return sm


def oracle_freqs(cfg, blend=False):
    if blend:
        return oracle.yarn_inv_freq(cfg.head_dim, cfg.rope_base, cfg.yarn_factor,
                                    cfg.yarn_orig_max_pos)
    return oracle.rope_inv_freq(cfg.head_dim, cfg.rope_base)


def host64(t):
    """Exact fp64 copy of a device/host tensor (bf16 and fp32 values)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_inputs(q, k, v):
    """What the oracle sees: fp32 inputs rounded to bf16 as the library does on
    entry, bf16 inputs as they are."""
    def conv(t):
        a = t.detach().float().cpu().numpy()
        if t.dtype == torch.float32:
            a = oracle.bf16_round(a)
        return a.astype(np.float64)
    return conv(q), conv(k), conv(v)


def build_cache(layer, k, v, upto):
    """Fill the layer's caches for tokens [0, upto) (one rope call per 32K)."""
    step = 32768
    for c0 in range(0, upto, step):
        c1 = min(upto, c0 + step)
        layer.append_kv(k[:, c0:c1], v[:, c0:c1], c0)


def compare(gpu, ref, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    d = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    print(f"[compare] max-abs {d.max():.3e} mean-abs {d.mean():.3e}")
    assert d.max() <= max_abs, f"max-abs {d.max():.3e} > {max_abs}"
    assert d.mean() <= mean_abs, f"mean-abs {d.mean():.3e} > {mean_abs}"
    return d.max(), d.mean()


def lse_compare(gpu, ref, tol=2e-2):
    """lse within tol (a scalar or one bound per row)."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    both_inf = np.isneginf(g) & np.isneginf(r)
    with np.errstate(invalid="ignore"):
        d = np.abs(np.where(both_inf, 0.0, g - r))
    assert np.all(d <= tol), f"lse max diff {d.max():.3e} (worst excess {np.max(d - tol):.3e})"
    return d.max()



# Estimate scores against fp64: every score within SCORE_REL of the largest
# score of its kind.  The scores are sums of row-softmax probabilities; the
# fp16 rounding of both QK^T operands (unit roundoff u = 2^-11) moves a logit
# l by at most about 2 u |l| (operands aligned), so a probability by that
# relative amount.  With unit-variance Q/K every score carries a relative
# error of about 2e-3 (measured 1.1e-3 .. 2.5e-3 on the scores above 1e-3 of
# the largest; 2e-4 .. 1.4e-3 of the largest score overall); the
# refinement-stress planting puts far-sink logits near 12 (2 u |l| ~
# 1.2e-2), measured 2.1e-3 of the largest score, hence its own bound.
SCORE_REL = 2e-3
SCORE_REL_LARGE_LOGITS = 4e-3
# Selections from GPU scores and from fp64 scores may disagree only between
# scores the rounding above can reorder: the fp64 gap between a swapped index
# and the fp64 boundary score must stay within twice the per-score relative
# error bound (NEAR_TIE_REL) of the boundary score.
NEAR_TIE_REL = 2 * 5e-3


def score_compare(got, ref, what, quiet=False, rel=SCORE_REL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = float(np.max(np.abs(ref)))
    d = np.abs(got - ref)
    if not quiet:
        big = ref > 1e-3 * scale
        rel_big = float(np.max(d[big] / ref[big])) if big.any() else 0.0
        print(f"  {what}: max |d| {d.max():.2e} = {d.max() / scale:.2e} of the largest score; "
              f"max relative error of scores above 1e-3 of it: {rel_big:.2e}", flush=True)
    assert d.max() <= rel * scale, f"{what}: max |d| {d.max():.3e} > {rel} x {scale:.3e}"
    return d.max() / scale


def near_tie_check(gpu_sel, ref_scores, k, what):
    """The GPU's selection (from its own scores) against the oracle's
    selection of the fp64 scores: every index in one set but not the other
    must be a near-tie of the fp64 boundary score."""
    ref = np.asarray(ref_scores, np.float64)
    sel = oracle.select_top(ref, k)
    diff = np.array(sorted(set(np.asarray(gpu_sel).tolist()) ^ set(sel.tolist())), np.int64)
    if diff.size == 0:
        print(f"  {what}: selections identical ({sel.size})", flush=True)
        return 0.0
    kth = float(np.min(ref[sel]))
    gap = float(np.max(np.abs(ref[diff] - kth)))
    scale = float(np.max(ref))
    print(f"  {what}: {diff.size // 2} swaps of {sel.size}; widest gap to the boundary "
          f"{gap:.2e} = {gap / kth:.2e} of the boundary score ({gap / scale:.2e} of the "
          f"largest)", flush=True)
    assert gap <= NEAR_TIE_REL * kth, f"{what}: disagreement {gap:.3e} is not a near-tie"
    return gap / kth


def _one_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def _run_job(job):
    fn, args = job
    return fn(*args)


def parallel_map(fn, arg_list, workers=12):
    """fn(*args) for every args tuple, in forked worker processes (CPU only:
    the workers run the numpy oracle and never touch the GPU), results in
    order.  Large read-only state (key contexts) must be built before the
    call; the workers inherit it instead of receiving it.  At most 12
    workers, which with the parent keeps the number of processes on the
    machine modest.  They end with os._exit (multiprocessing's own), so no
    GPU runtime teardown runs in them."""
    import multiprocessing as mp
    import os
    arg_list = list(arg_list)
    n = min(len(arg_list), workers, os.cpu_count() or 1)
    if n <= 1:
        return [fn(*a) for a in arg_list]
    with mp.get_context("fork").Pool(n, initializer=_one_thread) as pool:
        return pool.map(_run_job, [(fn, a) for a in arg_list], chunksize=1)


def critical_pair_total(verts, slashes, c0, c1):
    """Sum over rows i in [c0, c1) of |C_i|, C_i = {v in verts : v <= i} U
    {i - o : o in slashes, o <= i} (each key once), by inclusion and
    exclusion on the index sets: the verticals' rows, plus the slashes'
    rows, minus the (vertical, slash) pairs that name the same key of a row
    (v + o = i).  verts and slashes hold distinct indices."""
    v = np.unique(np.asarray(verts, dtype=np.int64))
    o = np.unique(np.asarray(slashes, dtype=np.int64))
    v = v[(v >= 0) & (v < c1)]
    o = o[(o >= 0) & (o < c1)]
    n_v = int(np.sum(c1 - np.maximum(v, c0)))
    n_s = int(np.sum(c1 - np.maximum(o, c0)))
    # pairs with c0 <= v + o < c1
    both = int(np.sum(np.searchsorted(o, c1 - v, side="left") -
                      np.searchsorted(o, c0 - v, side="left")))
    return n_v + n_s - both
