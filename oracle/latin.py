"""Latin-square layer schedules, in plain Python (test infrastructure, see ``oracle``).

Source: "Placement Is Free, Composition Is Not", sec. 1 and sec. 3.2: N mechanisms over N^2
layers arranged so that no mechanism repeats within a row or within a column; Table 7 prints the 4x4
proxy schedule row by row ("SGMF GMFS MFSG FSGM"), which is the cyclic left shift of its
first row, read row-major into layer order.
"""
from __future__ import annotations


def cyclic_square(base):
    """The N x N square whose row r is ``base`` rotated left by r: cell (r, c) holds
    base[(r + c) mod N]. Returned flat, row-major (layer l = r * N + c)."""
    n = len(base)
    return [base[(r + c) % n] for r in range(n) for c in range(n)]


def is_latin(n: int, sched) -> bool:
    """True iff the flat row-major schedule of n*n entries holds n distinct types and no
    type repeats within any row or within any column (so each row and each column holds
    every type)."""
    if n < 1 or len(sched) != n * n:
        return False
    symbols = set(sched)
    if len(symbols) != n:
        return False
    for r in range(n):
        if len(set(sched[r * n:(r + 1) * n])) != n:
            return False
    for c in range(n):
        if len({sched[r * n + c] for r in range(n)}) != n:
            return False
    return True
