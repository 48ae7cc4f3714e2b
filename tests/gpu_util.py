"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs."""

import math

import numpy as np
import torch

import oracle
import long_context_sparse_rope_amd as L

DEV = "cuda"

# Output bar for bf16 inputs with fp32 accumulation.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def rope_of(cfg, blend=False):
    return L.RopeConfig(base=cfg.rope_base, yarn_factor=cfg.yarn_factor,
                        orig_max_pos=cfg.yarn_orig_max_pos, freq_blend=blend)


def dca_of(cfg):
    return L.DcaConfig(cfg.dca_chunk, cfg.dca_local)


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

