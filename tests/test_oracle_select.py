"""Pins for the oracle's budget selection: the rounding table, brute force against
a full lexicographic sort, ties, and the candidate set. No GPU."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("n_full,s,expect", [
    (16, 0.25, 4),        # tiny workload: 4 of 16 pages
    (1024, 0.05, 52),     # 51.2 -> 52
    (1536, 0.05, 77),     # 76.8 -> 77
    (1000, 0.10, 100),    # 0.1 * 1000 in float64: the guard keeps 100
    (1024, 0.50, 512),
    (10, 1.0, 10),        # budget 1 keeps every page
    (10, 1e-6, 1),        # at least one page
    (0, 0.5, 0),          # no full page, nothing to choose
    (3, 0.34, 2),
])
def test_num_selected_table(n_full, s, expect):
    assert oracle.num_selected(n_full, s) == expect


def test_select_matches_full_sort_with_ties():
    rng = np.random.default_rng(11)
    B, MP, P = 6, 40, 16
    lens = np.array([0, 15, 16, 200, 639, 640], dtype=np.int32)
    S = rng.random((B, MP)).astype(np.float32)
    S[3, 2:9] = 0.5                      # a run of exact ties
    S[4, ::3] = S[4, 1]
    S[:, 38:] = 10.0                     # pages beyond the full pages must never win
    for s in (0.05, 0.25, 0.5, 1.0):
        sel = oracle.select_budget(S, lens, P, s)
        for b in range(B):
            nf = int(lens[b]) // P
            k = oracle.num_selected(nf, s)
            # lexsort: last key is primary -> (-score, index)
            order = np.lexsort((np.arange(nf), -S[b, :nf].astype(np.float64)))
            ref = np.sort(order[:k])
            np.testing.assert_array_equal(sel[b], ref)
            assert np.all(np.diff(sel[b]) > 0)
            assert sel[b].size == 0 or sel[b].max() < nf


def test_select_tie_break_prefers_lower_page():
    S = np.zeros((1, 8), dtype=np.float32)
    S[0, [1, 4, 6]] = 1.0
    sel = oracle.select_budget(S, np.array([128]), 16, 0.25)     # 2 of 8
    np.testing.assert_array_equal(sel[0], [1, 4])


def test_select_with_a_budget_per_row_is_the_scalar_selection_of_each_row():
    """One budget per row: each row equals the one-budget selection of that row alone
    (checked against the full sort), and equal budgets give the one-budget result."""
    rng = np.random.default_rng(12)
    B, MP, P = 7, 64, 16
    lens = np.array([0, 15, 100, 400, 777, 1000, 1024], dtype=np.int32)
    S = rng.random((B, MP)).astype(np.float32)
    S[4, 3:20] = 0.25                    # ties
    budgets = np.array([0.5, 0.05, 0.3, 0.07, 1.0, 0.125, 0.9], dtype=np.float64)
    sel = oracle.select_budget(S, lens, P, budgets)
    for b in range(B):
        nf = int(lens[b]) // P
        k = oracle.num_selected(nf, float(budgets[b]))
        order = np.lexsort((np.arange(nf), -S[b, :nf].astype(np.float64)))
        np.testing.assert_array_equal(sel[b], np.sort(order[:k]))
        np.testing.assert_array_equal(sel[b], oracle.select_budget(S[b:b + 1], lens[b:b + 1], P,
                                                                   float(budgets[b]))[0])
    same = oracle.select_budget(S, lens, P, np.full(B, 0.25))
    ref = oracle.select_budget(S, lens, P, 0.25)
    for b in range(B):
        np.testing.assert_array_equal(same[b], ref[b])


@pytest.mark.parametrize("s,expect", [(0.10, 100), (0.05, 50), (0.25, 250), (0.3, 300)])
def test_a_budget_per_row_rounds_as_the_scalar_budget(s, expect):
    """Per-row budgets are double values, rounded by the same rule as the scalar
    budget: 0.1 of 1000 full pages keeps 100 pages either way (a float32 0.1 would
    be 0.100000001 and keep 101)."""
    P, MP = 16, 1000
    lens = np.array([MP * P, MP * P], dtype=np.int32)
    S = np.random.default_rng(5).random((2, MP)).astype(np.float32)
    per_row = oracle.select_budget(S, lens, P, np.array([s, s]))
    scalar = oracle.select_budget(S, lens, P, s)
    for b in range(2):
        assert per_row[b].size == expect
        np.testing.assert_array_equal(per_row[b], scalar[b])
    assert oracle.num_selected(MP, float(np.float32(0.1))) == 101
