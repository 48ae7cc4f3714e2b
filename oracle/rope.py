"""RoPE, YaRN frequencies and the YaRN attention temperature (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

import math

import numpy as np


def bf16_round(x):
    """Round float32 values to the nearest bfloat16 (ties to even), as fp32.

    The library converts fp32 inputs to bf16 on entry; the oracle applies
    the same rounding to those inputs (the tiny fp32 config).  Rounding of
    rotated operands is a separate, optional mode of the oracle
    (KeyContext(operands="bf16" or "fp16")) that models an operand precision
    of the matrix cores; parity is asserted without it.
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return rounded.view(np.float32).reshape(a.shape)


def bf16_round64(x):
    """Round float64 values straight to the nearest bfloat16 (ties to even),
    returned as float64, with no float32 step in between.

    bfloat16 keeps 8 significant bits: with x = m 2^e and 1/2 <= |m| < 1,
    the result is round_half_even(256 m) 2^(e - 8).
    """
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.round(m * 256.0), e - 8)


def fp16_round64(x):
    """Round float64 values straight to the nearest IEEE binary16 (ties to
    even), returned as float64.  numpy converts float64 to float16 in one
    correctly rounded step (11 significant bits; subnormals below 2^-14,
    overflow to inf above 65504)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def rope_inv_freq(head_dim, base):
    """theta_p = base ** (-2p / D) for p = 0 .. D/2-1.

    [architecture overview] §2.4 code: inverse frequencies of the rotary
    embedding, one per rotated pair of dimensions.
    """
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    p = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * p / head_dim)


def yarn_inv_freq(head_dim, base, factor, orig_max_pos, beta_fast=32.0,
                  beta_slow=1.0):
    """YaRN "NTK-by-parts" frequency blend.

    [long-context blog] "YaRN実装" names the parameters (scale,
    original_max_pos, beta_fast=32, beta_slow=1) and the blend
    (1 - smooth) * f / scale + smooth * f; its code is garbled (it compares a
    wavelength with a frequency).  Reading: the published YaRN definition.
    For each pair p, r_p = orig_max_pos / wavelength_p is the number of turns
    the pair makes over the training length; gamma_p ramps linearly from 0 at
    r_p <= beta_slow to 1 at r_p >= beta_fast; the new frequency is
    theta_p * ((1 - gamma_p) / factor + gamma_p).  Fast pairs are kept,
    slow pairs are interpolated by 1/factor ([architecture overview] §2.2:
    the longest wavelengths are interpolated).  factor <= 1 returns theta.
    Pinned by three hand-worked pairs inside the ramp (tests/golden/
    yarn_ramp.txt) besides its end points and band sizes.
    """
    theta = rope_inv_freq(head_dim, base)
    if factor <= 1.0:
        return theta
    wavelength = 2.0 * math.pi / theta
    turns = float(orig_max_pos) / wavelength
    gamma = np.clip((turns - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    return theta * ((1.0 - gamma) / float(factor) + gamma)


def yarn_mscale(factor):
    """sqrt(1/t) = 0.1 ln(s) + 1 ([Qwen2.5-1M explainer] Length
    Extrapolation, YaRN attention scaling); s <= 1 means no scaling."""
    if factor <= 1.0:
        return 1.0
    return 0.1 * math.log(factor) + 1.0


def softmax_scale(head_dim, factor):
    """1 / (t * sqrt(D)) from softmax(q^T k / (t sqrt(D))) with
    sqrt(1/t) = mscale, i.e. mscale**2 / sqrt(D)."""
    return yarn_mscale(factor) ** 2 / math.sqrt(head_dim)


def rope_rotate(x, pos, inv_freq):
    """Rotate vectors x[..., D] at integer positions pos[...] (fp64).

    rotate_half convention ([architecture overview] §2.4 code:
    q * cos + rotate_half(q) * sin with emb = cat(freqs, freqs)): the pair
    (x_p, x_{p+D/2}) turns by the angle pos * theta_p,
        x'_p       = x_p cos - x_{p+D/2} sin
        x'_{p+D/2} = x_{p+D/2} cos + x_p sin.
    Angles are formed in float64 from the exact integer position.
    """
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)
    half = x.shape[-1] // 2
    if inv_freq.shape[-1] != half:
        raise ValueError("inv_freq length must be D/2")
    ang = pos[..., None] * inv_freq
    c = np.cos(ang)
    s = np.sin(ang)
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_apply(x, pos, inv_freq, scale=1.0, rotate=True):
    """What the standalone RoPE call produces (before its bf16 store):
    scale * R(pos) x, or scale * x when rotate is False."""
    y = rope_rotate(x, pos, inv_freq) if rotate else np.asarray(x, np.float64)
    return y * float(scale)
