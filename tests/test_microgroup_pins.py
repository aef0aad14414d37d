"""Pins of the TP micro-group oracle (oracle/microgroup_ref.py) against cases
worked by hand from the algorithm's steps and against the LPT makespan bound
(Graham): an LPT schedule on R machines is within 4/3 - 1/(3R) of the best
one, which brute force finds on small groups. CPU only."""
import itertools
import random

import pytest

from oracle import microgroup_ref as mg


def test_global_order_is_cost_then_id_descending():
    assert mg.global_order([3, 5, 3, 1, 5]) == [4, 1, 2, 0, 3]


def test_min_heap_solver_by_hand():
    """Costs by ID 4, 7, 1, 5, 3 on 2 ranks, taken as 7, 5, 4, 3, 1: 7 -> r0
    (a tie at 0 goes to the lower rank); 5 -> r1; 4 -> r1 (5 < 7); 3 -> r0
    (7 < 9); 1 -> r1 (9 < 10). Loads 10, 10."""
    costs = [4, 7, 1, 5, 3]
    items = [0, 1, 2, 3, 4]
    l_max, host = mg.min_heap_solver(items, costs, 2)
    assert host == [1, 0, 1, 1, 0]
    assert l_max == 10.0


def test_rollback_by_hand():
    """Costs 6, 5, 4, 3, 2, 2 (IDs 0..5), R = 2, C_max = 8.
    {6} ok (6); {6,5} -> 6 | 5 ok; {6,5,4} -> 6 | 9 > 8: close {6,5}, seed {4};
    {4,3} ok; {4,3,2}: 4 | 3+2 ok (5); {4,3,2,2}: 4+2 | 3+2 -> 6 | 5 ok."""
    costs = [6, 5, 4, 3, 2, 2]
    groups = mg.micro_groups(costs, 2, 8.0)
    assert [g for g, _ in groups] == [[0, 1], [2, 3, 5, 4]]
    # hosts: {6,5} -> r0, r1; {4,3,2(id5),2(id4)}: 4 -> r0, 3 -> r1, 2 -> r1 (3 < 4), 2 -> r0 (4 < 5)
    assert [h for _, h in groups] == [[0, 1], [0, 1, 1, 0]]


def test_a_tensor_heavier_than_the_capacity_forms_its_own_group():
    groups = mg.micro_groups([10, 3, 3], 2, 4.0)
    assert [g for g, _ in groups] == [[0], [2, 1]]


@pytest.mark.parametrize("seed", range(40))
def test_lpt_bound_against_brute_force(seed):
    rng = random.Random(seed)
    R = rng.choice([2, 3])
    costs = [rng.randint(1, 20) for _ in range(rng.randint(1, 7))]
    items = list(range(len(costs)))
    l_max, host = mg.min_heap_solver(items, costs, R)
    best = min(max(sum(c for c, a in zip(costs, asg) if a == r) for r in range(R))
               for asg in itertools.product(range(R), repeat=len(costs)))
    assert l_max <= (4 / 3 - 1 / (3 * R)) * best + 1e-9
    loads = [sum(c for c, h in zip(costs, host) if h == r) for r in range(R)]
    assert max(loads) == l_max


@pytest.mark.parametrize("seed", range(30))
def test_schedule_invariants(seed):
    rng = random.Random(100 + seed)
    R = rng.choice([1, 2, 4, 8])
    costs = [rng.choice([rng.randint(1, 100), rng.randint(1, 10 ** 6)]) for _ in range(rng.randint(1, 60))]
    c_max = rng.choice([max(costs), sum(costs) / R, max(costs) * 2.5])
    groups = mg.micro_groups(costs, R, c_max)
    ids = [i for g, _ in groups for i in g]
    assert sorted(ids) == list(range(len(costs)))                  # every tensor exactly once
    flat_order = mg.global_order(costs)
    assert sorted(ids, key=flat_order.index) == [i for i in flat_order]   # groups are runs of the global order
    pos = {p: k for k, p in enumerate(flat_order)}
    for g, h in groups:
        assert sorted(pos[p] for p in g) == list(range(min(pos[p] for p in g), max(pos[p] for p in g) + 1))
        loads = [0.0] * R
        for p, r in zip(g, h):
            loads[r] += costs[p]
        assert max(loads) <= c_max or len(g) == 1                   # the capacity, unless a lone oversize tensor
