"""The oracle's greedy head against its pins, and planted mistakes the pins must catch."""

import math

import numpy as np
import pytest

import head_pins as hp
import oracle


@pytest.mark.parametrize("check", hp.HEAD_CHECKS, ids=lambda c: c.__name__)
def test_head_pin(check):
    check(oracle.greedy_head)


def _variant(last_tie=False, nan_wins=False, count_ninf=False, no_norm=False, base2=False,
             nan_as_zero=False):
    def head(x):
        x = np.asarray(x, dtype=np.float64)
        if nan_as_zero:
            x = np.nan_to_num(x, nan=0.0, neginf=-np.inf)
        rows, V = x.shape
        tok = np.full(rows, -1)
        top = np.full(rows, np.nan)
        for r in range(rows):
            row = x[r]
            valid = ~np.isnan(row)
            if nan_wins and np.isnan(row).any():
                tok[r] = int(np.flatnonzero(np.isnan(row))[0])
                continue
            if not valid.any():
                continue
            m = row[valid].max()
            hits = np.flatnonzero(valid & (row == m))
            tok[r] = int(hits[-1] if last_tie else hits[0])
            if m == -math.inf:
                continue
            d = row[valid] - m
            e = np.exp2(d) if base2 else np.exp(d)
            if count_ninf:
                e = np.where(np.isneginf(row[valid]), 1.0, e)
            top[r] = 1.0 if no_norm else 1.0 / e.sum()
        return tok, top
    return head


MUTANTS = {
    "last_index_on_ties": _variant(last_tie=True),
    "nan_wins": _variant(nan_wins=True),
    "ninf_counted": _variant(count_ninf=True),
    "not_normalised": _variant(no_norm=True),
    "base2_exponent": _variant(base2=True),
    "nan_read_as_zero": _variant(nan_as_zero=True),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_head_pins_catch_mutant(name):
    fails = 0
    for check in hp.HEAD_CHECKS:
        try:
            check(MUTANTS[name])
        except AssertionError:
            fails += 1
    assert fails, f"head mutant {name} passed every pin"


def test_unmutated_variant_passes():
    for check in hp.HEAD_CHECKS:
        check(_variant())
