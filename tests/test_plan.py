"""The slot rule that include/mla.h documents for mla_decode_paged's partials,
as restated in tests/_plan.py (host logic, no GPU): every visible page of a row
lands in exactly one piece, slots are distinct and below num_splits, no piece
crosses a range border and no range holds more than W pages."""
import numpy as np
import pytest

from tests._plan import WORKGROUPS, header_pieces, row_pages


@pytest.mark.parametrize("S", [1, 2, 7, 16, 17, 64])
def test_header_rule_covers_rows_and_balances(S):
    g = np.random.default_rng(5)
    for rows in ([1024] * 16, [64] * 16, list(g.integers(0, 513, 64)), [0, 0, 3], [1], [260] * 1024,
                 list(g.integers(0, 40, 300))):
        p_tot, n_max = sum(rows), max(rows)
        plan = header_pieces(rows, S)
        W = -(-p_tot // WORKGROUPS) if p_tot else 1
        if S > 1 and p_tot:
            W = max(W, -(-(n_max - 1) // (S - 1)), 1)
        load = {}
        P = 0
        for nr, pieces in zip(rows, plan):
            covered = sorted(p for _, a, e in pieces for p in range(a, e))
            assert covered == list(range(nr))
            slots = [s_ for s_, _, _ in pieces]
            assert len(set(slots)) == len(slots) and all(0 <= s_ < S for s_ in slots)
            for s_, a, e in pieces:
                k = (P + a) // W if S > 1 else P // W
                assert k < WORKGROUPS
                if S > 1:
                    assert (P + e - 1) // W == k
                    assert s_ == k - P // W
                load[k] = load.get(k, 0) + (e - a)
            P += nr
        if S > 1 and load:
            assert max(load.values()) <= W


def test_header_rule_on_equal_rows_is_one_piece_per_range():
    plan = header_pieces([1024] * 16, 17)
    assert all(len(p) == 16 and [s for s, _, _ in p] == list(range(16)) for p in plan)
    assert all(e - a == 64 for p in plan for _, a, e in p)


def test_row_pages_follow_the_causal_rule():
    assert row_pages([0, 1, 64, 65, 130], 1) == [0, 1, 1, 2, 3]
    # two new tokens: query 0 sees L - 1 keys, query 1 sees L
    assert row_pages([65, 1], 2) == [1, 2, 0, 1]
