"""Pins of the oracle's DCA position maps (CPU only)."""

import os

import numpy as np
import pytest

import oracle
from tests import brute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _table(name):
    rows = {}
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if ":" in line:
            k, v = line.split(":")
            rows[int(k)] = [int(x) for x in v.split()]
        else:
            vals = [int(x) for x in line.split()]
            rows[vals[0]] = vals[1:]
    return rows


def test_maps_hand_worked_table():
    tab = _table("dca_positions_C8_W2.txt")
    tok = np.array(sorted(tab))
    m = oracle.dca_position_maps(tok, 8, 2)
    for key, col in (("pk", 0), ("intra", 1), ("succ", 2), ("inter", 3)):
        assert m[key].tolist() == [tab[t][col] for t in tok], key


def test_relative_positions_hand_worked():
    tab = _table("dca_relpos_C8_W2.txt")
    for i, rel in tab.items():
        got = oracle.relative_positions(i, np.arange(i + 1), 8, 2)
        assert got.tolist() == rel, i


@pytest.mark.parametrize("chunk,local,n", [(8, 2, 40), (16, 4, 70), (256, 64, 1024), (12, 0, 50)])
def test_relative_positions_brute_force(chunk, local, n):
    for i in range(n):
        js = np.arange(i + 1)
        got = oracle.relative_positions(i, js, chunk, local)
        ref = [brute.rel_position_dca(i, int(j), chunk, local) for j in js]
        assert got.tolist() == ref
        # no distance reaches the training length C
        assert got.min() >= 0 and got.max() <= chunk - 1


def test_successive_window_continuity():
    chunk, local = 256, 64
    s = chunk - local
    for i in range(s, 3 * s):
        ip = i % s
        js = np.arange(max(0, (i // s - 1) * s), (i // s) * s)   # previous chunk
        rel = oracle.relative_positions(i, js, chunk, local)
        if ip < local:
            assert rel.tolist() == (i - js).tolist()
        else:
            assert rel.tolist() == (chunk - 1 - js % s).tolist()


def test_dca_reduces_to_causal_when_seq_within_chunk():
    """seq <= C and W <= C/2: every causal relative position is i - j."""
    for chunk, local in ((256, 64), (256, 128), (64, 16)):
        for i in range(chunk):
            js = np.arange(i + 1)
            assert oracle.relative_positions(i, js, chunk, local).tolist() == (i - js).tolist()


def test_dca_off_is_identity():
    tok = np.arange(100)
    m = oracle.dca_position_maps(tok, 0, 0)
    for key in m:
        assert m[key].tolist() == tok.tolist()
    assert oracle.relative_positions(77, tok[:78], 0, 0).tolist() == (77 - tok[:78]).tolist()


def test_large_positions():
    chunk, local = 262144, 32768
    s = chunk - local
    i = 1048575
    js = np.array([0, 5, s - 1, s, 2 * s + 7, 3 * s, 4 * s, i])
    rel = oracle.relative_positions(i, js, chunk, local)
    ref = [brute.rel_position_dca(i, int(j), chunk, local) for j in js]
    assert rel.tolist() == ref
    assert rel.max() <= chunk - 1
