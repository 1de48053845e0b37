"""Pins of the Latin-square schedule definitions (CPU only).

Source: "Placement Is Free, Composition Is Not", sec. 1 and sec. 3.2 (no type repeats within a
row or a column), Table 7 (the printed 4x4 proxy schedule and its counter-examples).
"""
import itertools
import os

import pytest

from oracle import latin

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "table7_schedules.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((parts[0], parts[1] == "1", "".join(parts[2:])))
    return rows


def test_table7_latin_row_is_the_cyclic_square_of_its_first_row():
    arms = {name: seq for name, _, seq in _golden()}
    assert "".join(latin.cyclic_square(list("SGMF"))) == arms["latin"]


@pytest.mark.parametrize("name,expect,seq", _golden())
def test_table7_arms(name, expect, seq):
    assert len(seq) == 16
    assert latin.is_latin(4, list(seq)) is expect


def test_three_by_three_stack_rows():
    assert latin.cyclic_square(["F", "S", "D"]) == list("FSDSDFDFS")


@pytest.mark.parametrize("n", range(1, 12))
def test_cyclic_square_is_latin_for_every_n(n):
    assert latin.is_latin(n, latin.cyclic_square(list(range(n))))


def _count_latin(n):
    perms = list(itertools.permutations(range(n)))
    count = 0
    for rows in itertools.product(perms, repeat=n):
        if latin.is_latin(n, [x for r in rows for x in r]):
            count += 1
    return count


def test_count_of_latin_squares_matches_known_values():
    # Number of Latin squares of order n over a fixed n-symbol set: 1, 2, 12, 576.
    assert [_count_latin(n) for n in (1, 2, 3)] == [1, 2, 12]
    assert _count_latin(4) == 576


def test_count_over_all_3x3_grids():
    # Among all 3^9 grids over {0, 1, 2}, exactly 12 are Latin.
    n = sum(latin.is_latin(3, list(g)) for g in itertools.product(range(3), repeat=9))
    assert n == 12


def test_rejects_wrong_sizes_and_symbol_counts():
    assert not latin.is_latin(0, [])
    assert not latin.is_latin(2, [0, 1, 1])
    assert not latin.is_latin(2, [0, 1, 2, 3])       # four symbols in a 2x2 grid
    assert not latin.is_latin(2, [0, 0, 1, 1])
