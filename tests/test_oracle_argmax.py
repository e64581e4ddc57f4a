"""Pins for the oracle's greedy argmax (CPU only): hand-worked rows, and
numpy.argmax (first occurrence of the maximum, first NaN) as an independent
library routine on random rows with many exact ties."""

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("row,want", [
    ([1.0, 3.0, 3.0, 2.0], 1),            # exact tie: lower index
    ([-5.0, -2.0, -2.0], 1),              # all negative
    ([-0.0, 0.0], 0),                     # -0 equals +0
    ([0.0, -0.0, -1.0], 0),
    ([1.0, float("nan"), 5.0, float("nan")], 1),   # first NaN wins
    ([float("nan"), 7.0], 0),
    ([float("-inf"), -1e30], 1),
    ([float("inf"), float("inf")], 0),
    ([2.0], 0),
])
def test_hand_rows(row, want):
    assert oracle.greedy_argmax(np.array(row)).tolist() == [want]


def test_matches_numpy_first_occurrence():
    rng = np.random.default_rng(11)
    for trial in range(30):
        n = int(rng.integers(1, 300))
        # Few distinct values, so most rows have exact ties at the maximum.
        row = rng.integers(-4, 5, size=n).astype(np.float64) * 0.5
        if trial % 5 == 0:
            row[rng.integers(0, n, size=max(1, n // 50))] = np.nan
        assert oracle.greedy_argmax(row)[0] == int(np.argmax(row)), trial


def test_rows_independent():
    a = np.array([[0.0, 1.0, 1.0], [3.0, 3.0, 0.0], [-1.0, -1.0, -0.5]])
    assert oracle.greedy_argmax(a).tolist() == [1, 0, 2]
