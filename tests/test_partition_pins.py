"""Pins of the DP static-partition oracle (oracle/partition_ref.py), against
the pages' worked example and small cases worked by hand from the algorithm's
steps. CPU only."""
import random

import pytest

from oracle import partition_ref as pr


def test_start_index_worked_example():
    """A parameter starting at element 1,048,577 with stride S = 1,048,576
    belongs to rank 1's slice (Canzona analysis page, section 3.4, Paradigm 3),
    and so does everything of it that reaches past 2 S."""
    S = 1_048_576
    bucket = [S + 1, S, 2 * S - 1]            # starts: 0, S + 1, 2 S + 1; |B| = 4 S
    cuts = pr.static_partition([bucket], 4)[0]
    owner = [r for j in range(3) for r in range(4) if cuts[r] <= j < cuts[r + 1]]
    assert owner == [0, 1, 2]
    assert cuts == [0, 1, 2, 3, 3]            # rank 3 starts no parameter


def test_static_rule_last_rank_and_uneven_stride():
    # |B| = 10 over 3 ranks: S = 10/3; starts 0, 3, 4, 9 -> ranks 0, 0, 1, 2
    cuts = pr.static_partition([[3, 1, 5, 1]], 3)[0]
    assert cuts == [0, 2, 3, 4]


def test_alpha_one_fills_the_deficit_and_ties_go_to_the_earlier_boundary():
    """R = 2, buckets [6] and [1, 1, 1, 1], mu = 5. LPT takes [6] first: even
    shares, C = 3 sits halfway between boundaries 0 and 6, the tie picks 0, so
    rank 1 takes it (L = [0, 6]). Then d = [5, 0] and alpha = 1 gives rank 0
    the whole second bucket: L = [4, 6]."""
    loads = [[6], [1, 1, 1, 1]]
    cuts = pr.alpha_balanced(loads, 2, 1.0)
    assert cuts == [[0, 0, 1], [0, 4, 4]]
    assert pr.rank_loads(loads, cuts, 2) == [4.0, 6.0]
    assert pr.load_balance_ratio([4.0, 6.0]) == pytest.approx(1.2)
    # alpha = 0 ignores the deficit: the second bucket is split evenly
    cuts0 = pr.alpha_balanced(loads, 2, 0.0)
    assert cuts0 == [[0, 0, 1], [0, 2, 4]]
    assert pr.rank_loads(loads, cuts0, 2) == [2.0, 8.0]


def test_alpha_blend():
    """R = 2, buckets [5, 1, 1, 1] and [2, 2], mu = 6. First bucket: C = 4,
    boundary 1 (prefix 5) is closest: L = [5, 3]. Second: d = [1, 3],
    fill = [1/4, 3/4]. alpha = 0.5: v0 = 3/8, C = 1.5, boundary 1 (prefix 2);
    alpha = 1: C = 1, a tie between prefixes 0 and 2, boundary 0."""
    loads = [[5, 1, 1, 1], [2, 2]]
    assert pr.alpha_balanced(loads, 2, 0.5) == [[0, 1, 4], [0, 1, 2]]
    assert pr.alpha_balanced(loads, 2, 1.0) == [[0, 1, 4], [0, 0, 2]]
    assert pr.alpha_balanced(loads, 2, 0.0) == [[0, 1, 4], [0, 1, 2]]


def test_lpt_order_visits_the_heaviest_bucket_first():
    """Buckets [1] and [2, 2, 2], R = 2, alpha = 1. Heaviest first: the big
    bucket is cut at a tie (C = 3 between prefixes 2 and 4) at boundary 1,
    then the deficit sends [1] to rank 0. In index order the result would be
    [[0, 0, 1], [0, 2, 3]] instead."""
    loads = [[1], [2, 2, 2]]
    assert pr.alpha_balanced(loads, 2, 1.0) == [[0, 1, 1], [0, 1, 3]]


def test_deficits_can_leave_a_rank_empty_handed():
    """Buckets [2]*6 and [3, 3] over 3 ranks: [4, 4, 4] after the first, then
    the cumulative targets 2 and 4 both pick boundary 1 of [3, 3]: [7, 4, 7]."""
    loads = [[2] * 6, [3, 3]]
    cuts = pr.alpha_balanced(loads, 3, 1.0)
    assert cuts == [[0, 2, 4, 6], [0, 1, 1, 2]]
    assert pr.rank_loads(loads, cuts, 3) == [7.0, 4.0, 7.0]


def test_objectives():
    loads = [[6], [1, 1, 1, 1]]
    cuts = [[0, 0, 1], [0, 4, 4]]
    j_dp, j_comm = pr.objectives(loads, loads, cuts, 2)
    assert j_dp == 1.0                 # |4 - 5| and |6 - 5|
    assert j_comm == 3.0 + 3.0 + 2.0 + 2.0


@pytest.mark.parametrize("seed", range(20))
def test_invariants_on_random_instances(seed):
    rng = random.Random(seed)
    R = rng.choice([1, 2, 3, 8, 32])
    buckets = [[rng.randint(1, 10 ** rng.randint(1, 7)) for _ in range(rng.randint(1, 12))]
               for _ in range(rng.randint(1, 9))]
    for alpha in (0.0, 0.3, 1.0):
        for cuts in (pr.alpha_balanced(buckets, R, alpha), pr.static_partition(buckets, R)):
            for b, c in zip(buckets, cuts):
                assert len(c) == R + 1 and c[0] == 0 and c[R] == len(b)
                assert all(c[r] <= c[r + 1] for r in range(R))      # monotone, on parameter boundaries
            tot = pr.rank_loads(buckets, cuts, R)
            assert sum(tot) == sum(sum(b) for b in buckets)          # every parameter owned exactly once
