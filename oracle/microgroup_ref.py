"""Plain CPU oracle of the TP micro-group schedule: the global LPT sort, the
greedy packing with rollback, and the min-heap host-rank assignment
(Algorithms 2 to 4).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py`` may import this module; the library never does, and this module
imports nothing from the library.

Source: Canzona analysis page (paper-graph-ui), section 3.4, "The TP
Hierarchical Partitioning and Scheduling (Micro-Group Construction)":
* Phase 1: every tensor sorted by (cost, ID), descending;
* Phase 2: walk the sorted tensors, tentatively add each to the current
  group, assign the group's tensors to the R host ranks with the min-heap
  solver, accept the tensor if the largest rank load stays within C_max, and
  otherwise close the current group and start the next one with the tensor;
* the min-heap solver: the group's tensors by cost, descending, each given to
  the least-loaded rank (a heap of (load, rank)).

Readings where the pages leave a step open:
* the tensor that triggers a rollback becomes the first member of the new
  group unconditionally, and the walk moves on (a tensor heavier than C_max
  alone then forms a group by itself instead of being retried forever);
* the solver's own sort keeps the global order among tensors of equal cost,
  and the heap breaks equal loads by the lower rank index;
* the descending (cost, ID) sort puts the larger ID first among equal costs.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple


def global_order(costs: Sequence[float]) -> List[int]:
    """Tensor indices (IDs) sorted by (cost, ID), descending."""
    return sorted(range(len(costs)), key=lambda i: (costs[i], i), reverse=True)


def min_heap_solver(items: Sequence[int], costs: Sequence[float], ranks: int) -> Tuple[float, List[int]]:
    """LPT on R ranks: items by cost, descending (stable), each to the rank of
    least load (lowest index on a tie). Returns (largest load, host rank of
    each item, in the order of ``items``)."""
    order = sorted(range(len(items)), key=lambda j: -costs[items[j]])   # stable
    load = [0.0] * ranks
    host = [0] * len(items)
    for j in order:
        best = min(range(ranks), key=lambda r: (load[r], r))
        host[j] = best
        load[best] += float(costs[items[j]])
    return max(load), host


def micro_groups(costs: Sequence[float], ranks: int, c_max: float) -> List[Tuple[List[int], List[int]]]:
    """The micro-group sequence: a list of (tensor IDs, their host ranks)."""
    groups: List[List[int]] = []
    curr: List[int] = []
    for p in global_order(costs):
        test = curr + [p]
        l_max, _ = min_heap_solver(test, costs, ranks)
        if l_max <= c_max or not curr:
            curr = test
        else:
            groups.append(curr)
            curr = [p]
    if curr:
        groups.append(curr)
    return [(g, min_heap_solver(g, costs, ranks)[1]) for g in groups]
