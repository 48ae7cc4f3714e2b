"""Pins of the oracle's RoPE / YaRN arithmetic (CPU only)."""

import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append([float(x) for x in line.split()])
    return out


def test_rope_hand_worked_example():
    inv = oracle.rope_inv_freq(4, 100.0)
    np.testing.assert_allclose(inv, [1.0, 0.1], rtol=0, atol=1e-15)
    for row in _rows("rope_d4_example.txt"):
        pos, x, y = row[0], row[1:5], row[5:9]
        got = oracle.rope_rotate(np.array(x), pos, inv)
        np.testing.assert_allclose(got, y, rtol=0, atol=1e-15)


def test_inv_freq_geometric():
    for d, base in ((64, 1e4), (128, 1e7)):
        th = oracle.rope_inv_freq(d, base)
        assert th[0] == 1.0
        np.testing.assert_allclose(th[1:] / th[:-1], base ** (-2.0 / d), rtol=1e-13)
        assert th.shape == (d // 2,)


def _complex_rotate(x, pos, theta):
    """Independent form: z_p = x_p + i x_{p+D/2} turns by exp(i pos theta_p)."""
    h = x.shape[-1] // 2
    z = x[..., :h] + 1j * x[..., h:]
    z = z * np.exp(1j * np.asarray(pos, np.float64)[..., None] * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_matches_complex_form():
    rng = np.random.default_rng(0)
    th = oracle.rope_inv_freq(128, 1e7)
    x = rng.normal(size=(50, 128))
    pos = rng.integers(0, 1 << 20, size=50)
    np.testing.assert_allclose(oracle.rope_rotate(x, pos, th),
                               _complex_rotate(x, pos, th), atol=1e-12)


def test_rope_identity_norm_and_composition():
    rng = np.random.default_rng(1)
    th = oracle.rope_inv_freq(64, 1e4)
    x = rng.normal(size=(8, 64))
    np.testing.assert_array_equal(oracle.rope_rotate(x, np.zeros(8), th), x)
    y = oracle.rope_rotate(x, np.arange(8) * 977, th)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    a, b = 1234, 55555
    np.testing.assert_allclose(
        oracle.rope_rotate(oracle.rope_rotate(x, a, th), b, th),
        oracle.rope_rotate(x, a + b, th), atol=1e-11)


def test_rope_relative_position_property():
    """q_m . k_n depends only on m - n (long-context blog, RoPE原理の復習)."""
    rng = np.random.default_rng(2)
    th = oracle.rope_inv_freq(128, 1e7)
    q, k = rng.normal(size=128), rng.normal(size=128)
    ref = oracle.rope_rotate(q, 700, th) @ oracle.rope_rotate(k, 300, th)
    for shift in (1, 4096, 262143, 1 << 20):
        got = oracle.rope_rotate(q, 700 + shift, th) @ oracle.rope_rotate(k, 300 + shift, th)
        assert abs(got - ref) < 1e-9
    # and it does change with the distance
    other = oracle.rope_rotate(q, 701, th) @ oracle.rope_rotate(k, 300, th)
    assert abs(other - ref) > 1e-6


def test_yarn_temperature_closed_form():
    for s, m, inv_t in _rows("yarn_temperature.txt"):
        assert oracle.yarn_mscale(s) == pytest.approx(m, abs=1e-15)
        assert oracle.yarn_mscale(s) ** 2 == pytest.approx(inv_t, abs=1e-15)
        assert oracle.softmax_scale(128, s) == pytest.approx(inv_t / math.sqrt(128), abs=1e-15)


def test_yarn_blend_end_points_and_ramp():
    d, base, L = 128, 1e7, 262144
    th = oracle.rope_inv_freq(d, base)
    assert np.array_equal(oracle.yarn_inv_freq(d, base, 1.0, L), th)
    for s in (2.0, 4.0):
        y = oracle.yarn_inv_freq(d, base, s, L)
        turns = L * th / (2 * math.pi)
        fast = turns >= 32.0
        slow = turns <= 1.0
        mid = ~fast & ~slow
        np.testing.assert_array_equal(y[fast], th[fast])
        np.testing.assert_allclose(y[slow], th[slow] / s, rtol=1e-15)
        ratio = y[mid] / th[mid]
        assert np.all((ratio > 1 / s) & (ratio < 1))
        # the kept fraction grows with the number of turns
        assert np.all(np.diff(ratio[np.argsort(turns[mid])]) > 0)
        # band sizes for base 1e7, D = 128, L = 262144, worked from
        # theta_p = 1e7^(-p/64): turns_p >= 32 <=> p <= 28.6; <= 1 <=> p >= 43.2
        assert (fast.sum(), mid.sum(), slow.sum()) == (29, 14, 21)


def test_yarn_ramp_hand_worked():
    """Three pairs inside the ramp (base 1e7, D 128, s 4, L 262,144), worked
    by hand step by step in tests/golden/yarn_ramp.txt."""
    y = oracle.yarn_inv_freq(128, 1e7, 4.0, 262144, beta_fast=32.0, beta_slow=1.0)
    th = oracle.rope_inv_freq(128, 1e7)
    for p, theta, gamma, theta_new in _rows("yarn_ramp.txt"):
        p = int(p)
        assert th[p] == pytest.approx(theta, rel=1e-14)
        assert y[p] == pytest.approx(theta_new, rel=1e-13)
        # the kept fraction of the frequency is (1 - gamma) / s + gamma
        assert y[p] / th[p] == pytest.approx((1 - gamma) / 4 + gamma, rel=1e-13)


def test_bf16_round_ties_and_library():
    one = np.float32(1.0)
    cases = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.0e38, 1e-40],
                     dtype=np.float32)
    got = oracle.bf16_round(cases)
    assert got[0] == one and got[1] == one          # tie -> even mantissa
    assert got[2] == np.float32(1 + 2 ** -6)        # tie -> even (upward)
    assert got[3] == -one
    rng = np.random.default_rng(3)
    x = (rng.normal(size=10000) * 10.0 ** rng.integers(-5, 5, 10000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(oracle.bf16_round(x), ref)


def test_bf16_round64_ties_and_library():
    """Direct fp64 -> bf16 rounding: the same ties as the fp32 path, the same
    result as torch on float32-representable values, and no double rounding
    on values that lie just off a tie in fp64."""
    got = oracle.bf16_round64(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0]))
    assert got.tolist() == [1.0, 1 + 2 ** -6, -1.0, 0.0]
    rng = np.random.default_rng(5)
    x = (rng.normal(size=10000) * 10.0 ** rng.integers(-5, 5, 10000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    np.testing.assert_array_equal(oracle.bf16_round64(x.astype(np.float64)), ref)
    # just above a tie in fp64, but a tie once squeezed through fp32 first
    y = 1 + 2 ** -8 + 2 ** -40
    assert oracle.bf16_round64(np.array([y]))[0] == 1 + 2 ** -7
    assert oracle.bf16_round(np.array([y], dtype=np.float32))[0] == 1.0
    # every result has at most 8 significant bits and lies within half an ulp
    z = rng.normal(size=5000) * 3.0
    r = oracle.bf16_round64(z)
    m, e = np.frexp(r)
    assert np.all(m * 256 == np.round(m * 256))
    assert np.all(np.abs(r - z) <= np.ldexp(1.0, np.frexp(z)[1] - 9))
