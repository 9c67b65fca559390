"""CPU checks of the SubBlock parity machinery itself (no GPU).

The GPU tests accept a kept list when it is valid against the oracle's scores
within error bounds and a top-keep set of the kernel's own scores.  Here the
oracle's own selection must pass those checks, and selections with a planted
mistake (a dropped block swapped for a lower-scoring one, a tie resolved to
the higher index, a repeated or unsorted index) must fail them.
"""
import numpy as np
import pytest

import oracle
from subblock_checks import (check_kept_lists, check_top_set_of_own_scores, check_valid_against_oracle,
                             pool_bound, score_bound, set_agreement)
from synthetic_inputs import bits, correlated_heads


@pytest.fixture(scope="module")
def routed():
    q = correlated_heads((1, 64 * 9 + 5, 2, 32), seed=3)
    k = correlated_heads((1, 64 * 9 + 5, 2, 32), seed=4)
    qp, kp, s, kept = oracle.subblock_route(bits(q), bits(k), 0.6)
    return q, qp, kp, s, kept


def test_oracle_selection_passes(routed):
    q, qp, kp, s, kept = routed
    nb, keep = s.shape[-1], kept.shape[-1]
    assert keep == oracle.subblock_keep(nb, 0.6) == 4
    check_kept_lists(kept, nb, keep)
    check_valid_against_oracle(kept, s, score_bound(qp, kp))
    check_top_set_of_own_scores(kept, s)
    assert set_agreement(kept, kept, nb) == 1.0
    assert np.all(pool_bound(bits(q), qp) > 0)


def test_planted_selection_mistakes_fail(routed):
    _, qp, kp, s, kept = routed
    nb = s.shape[-1]
    e = score_bound(qp, kp)
    row = (0, 1, 3)
    order = np.argsort(-s[row], kind="stable")
    worst_kept, best_dropped, worst = order[kept.shape[-1] - 1], order[kept.shape[-1]], order[-1]
    # swap the weakest kept block for the lowest-scoring block
    bad = kept.copy()
    bad[row] = np.sort(np.where(kept[row] == worst_kept, worst, kept[row]))
    with pytest.raises(AssertionError):
        check_valid_against_oracle(bad, s, e)
    with pytest.raises(AssertionError):
        check_top_set_of_own_scores(bad, s)
    assert set_agreement(bad, kept, nb) < 1.0
    # make the weakest kept block and the best dropped block tie: keeping the
    # lower index of the two passes, keeping the higher one must fail
    s2 = s.copy()
    s2[row][best_dropped] = s2[row][worst_kept]
    lo, hi = sorted((int(worst_kept), int(best_dropped)))
    rest = np.setdiff1d(kept[row], [worst_kept])
    tie_ok, tie_bad = kept.copy(), kept.copy()
    tie_ok[row] = np.sort(np.append(rest, lo))
    tie_bad[row] = np.sort(np.append(rest, hi))
    check_top_set_of_own_scores(tie_ok, s2)
    with pytest.raises(AssertionError):
        check_top_set_of_own_scores(tie_bad, s2)
    # a repeated index and an unsorted list
    rep = kept.copy()
    rep[row][1] = rep[row][0]
    with pytest.raises(AssertionError):
        check_kept_lists(rep, nb, kept.shape[-1])
    uns = kept.copy()
    uns[row] = uns[row][::-1]
    with pytest.raises(AssertionError):
        check_kept_lists(uns, nb, kept.shape[-1])
