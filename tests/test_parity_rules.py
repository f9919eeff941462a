"""CPU checks of the token comparison rule in tests/parity.py: a near-tie
(GPU token != the oracle's selection on the oracle's own row) passes only
when the GPU row's deviation at the two columns explains the gap, and for
bf16 greedy rows when the gap is at most one bf16 ulp."""
import numpy as np
import pytest

from rank_markov_draft_amd import workloads as wl
from tests import parity


def rows_with(values):
    row = np.full(16, -1.0, np.float32)
    for i, v in values.items():
        row[i] = v
    return wl.to_bf16_bits(row)[None, :]


def test_one_ulp_flip_is_a_counted_near_tie():
    o = rows_with({3: 4.0 - 2.0 ** -6, 7: 4.0})     # oracle: 7 wins by one bf16 ulp
    g = rows_with({3: 4.0, 7: 4.0})                 # GPU row flipped column 3 up by one ulp: 3 wins the tie
    rep = parity.check_tokens(np.array([3]), g, o, 0.0, 0, [0], [0])
    assert rep.near_ties == 1 and rep.max_tie_gap == 2.0 ** -6


def test_unexplained_gap_fails():
    o = rows_with({3: 3.0, 7: 4.0})                 # a gap of 1.0, far beyond one ulp
    g = rows_with({3: 4.5, 7: 4.0})
    with pytest.raises(AssertionError, match="gap"):
        parity.check_tokens(np.array([3]), g, o, 0.0, 0, [0], [0])


def test_token_must_be_argmax_of_its_own_row():
    o = rows_with({3: 4.0, 7: 4.0})
    with pytest.raises(AssertionError, match="first argmax"):
        parity.check_tokens(np.array([7]), o, o, 0.0, 0, [0], [0])


def test_temperature_gap_needs_a_deviation():
    from oracle import oracle as orc
    row = np.zeros(16, np.float32)
    row[5] = 2.0
    T, seed = 0.7, 11
    o = wl.to_bf16_bits(row)[None, :]
    t_ref = orc.select_token(o[0], T, seed)[0]
    # a GPU row equal to the oracle's cannot select anything else
    rep = parity.check_tokens(np.array([t_ref]), o, o, T, seed, [0], [0])
    assert rep.near_ties == 0
    # raising another column far enough makes the GPU pick it: gap explained by the deviation
    other = (t_ref + 1) % 16
    g = row.copy()
    g[other] = 40.0
    gb = wl.to_bf16_bits(g)[None, :]
    t_g = orc.select_token(gb[0], T, seed)[0]
    assert t_g == other
    rep = parity.check_tokens(np.array([t_g]), gb, o, T, seed, [0], [0])
    assert rep.near_ties == 1
