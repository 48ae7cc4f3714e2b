"""Brute-force references for the oracle pins: pure Python loops, complex
numbers for the rotation and math.fsum for every sum.  Written from the
definitions independently of oracle/ (no import from it)."""

import cmath
import math


def inv_freq(d, base):
    return [base ** (-2.0 * p / d) for p in range(d // 2)]


def rel_position_dca(i, j, chunk, local):
    """Relative position of the pair (i, j), j <= i, stated pattern by pattern:
    same chunk -> i - j; adjacent chunk -> i - j inside the local window of
    the query's chunk, else (C-1) - (j mod S); farther -> (C-1) - (j mod S)."""
    if chunk == 0:
        return i - j
    s = chunk - local
    ci, cj = i // s, j // s
    if ci == cj:
        return i - j
    if ci - cj == 1 and (i - ci * s) < local:
        return i - j
    return (chunk - 1) - (j - cj * s)


def rope_dot(q, k, rel, freqs):
    """<R(a) q, R(b) k> with a - b = rel, via complex pairs z = x_p + i x_{p+D/2}:
    Re sum_p conj(z_k) z_q exp(i rel theta_p)."""
    h = len(q) // 2
    terms = []
    for p in range(h):
        zq = complex(q[p], q[p + h])
        zk = complex(k[p], k[p + h])
        terms.append((zk.conjugate() * zq * cmath.exp(1j * rel * freqs[p])).real)
    return math.fsum(terms)


def softmax_attend(logits, values):
    if not logits:
        return [0.0] * len(values[0]) if values else [], -math.inf
    m = max(logits)
    e = [math.exp(x - m) for x in logits]
    z = math.fsum(e)
    d = len(values[0])
    out = [math.fsum(e[a] * values[a][c] for a in range(len(e))) / z for c in range(d)]
    return out, m + math.log(z)


def attention_row(q, i, K, V, keys, freqs, scale, chunk, local):
    lg = [scale * rope_dot(q, K[j], rel_position_dca(i, j, chunk, local), freqs) for j in keys]
    vals = [V[j] for j in keys]
    if not keys:
        return [0.0] * len(V[0]), -math.inf
    return softmax_attend(lg, vals)


def estimate(qrows, rows, K, n_keys, freqs, scale):
    """Vertical and slash sums of row softmax probabilities, continuous positions."""
    v = [0.0] * n_keys
    s_terms = [[] for _ in range(n_keys)]
    v_terms = [[] for _ in range(n_keys)]
    for a, r in enumerate(rows):
        lg = [scale * rope_dot(qrows[a], K[j], r - j, freqs) for j in range(r + 1)]
        m = max(lg)
        e = [math.exp(x - m) for x in lg]
        z = math.fsum(e)
        for j in range(r + 1):
            p = e[j] / z
            v_terms[j].append(p)
            s_terms[r - j].append(p)
    return [math.fsum(t) for t in v_terms], [math.fsum(t) for t in s_terms]
