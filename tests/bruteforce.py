"""Brute-force attention at 50 significant digits with the standard-library ``decimal``.

An independent, matrix-form statement of the mixer layer used to pin the fp64 oracle on
tiny inputs: it materialises the whole L x L score matrix, builds the visibility mask as a
0/1 band matrix, and normalises exp(S) over visible entries without the max shift (decimal's
exponent range cannot overflow here). Nothing is shared with the oracle's C loops.

Semantics ("Placement Is Free, Composition Is Not", Table 1 and sec. 8): causal keys j <= i;
the sliding window keeps i - j < W; differential subtracts the second half-width map,
weighted by lambda, from the first, applied to full-width values.
"""
from __future__ import annotations

from decimal import Decimal, getcontext


def _dec_matrix(a):
    return [[Decimal(float(x)) for x in row] for row in a]


def _mask(L, variant, window):
    m = [[0] * L for _ in range(L)]
    for i in range(L):
        for j in range(L):
            if j > i:
                continue
            if variant == "sliding" and i - j >= window:
                continue
            m[i][j] = 1
    return m


def _probs(q, k, cols, scale, mask):
    L = len(q)
    s = [[sum((q[i][c] * k[j][c] for c in cols), Decimal(0)) * scale for j in range(L)]
         for i in range(L)]
    p = []
    for i in range(L):
        e = [s[i][j].exp() if mask[i][j] else Decimal(0) for j in range(L)]
        z = sum(e, Decimal(0))
        p.append([x / z for x in e])
    return p


def attention_decimal(q, k, v, variant: str, window: int = 0, lam: float = 0.0,
                      prec: int = 50):
    """One head: q, k, v are [L][d] nested sequences of floats. Returns [L][d] floats."""
    getcontext().prec = prec
    qd, kd, vd = _dec_matrix(q), _dec_matrix(k), _dec_matrix(v)
    L, d = len(qd), len(qd[0])
    mask = _mask(L, variant, window)
    if variant == "differential":
        half = d // 2
        scale = Decimal(1) / Decimal(half).sqrt()
        p1 = _probs(qd, kd, range(0, half), scale, mask)
        p2 = _probs(qd, kd, range(half, d), scale, mask)
        lamd = Decimal(float(lam))
        p = [[p1[i][j] - lamd * p2[i][j] for j in range(L)] for i in range(L)]
    else:
        scale = Decimal(1) / Decimal(d).sqrt()
        p = _probs(qd, kd, range(d), scale, mask)
    out = [[float(sum((p[i][j] * vd[j][c] for j in range(L)), Decimal(0))) for c in range(d)]
           for i in range(L)]
    return out
