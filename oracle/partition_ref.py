"""Plain CPU oracle of the DP static partition: the Start_Index ownership rule
and the alpha-Balanced Greedy LPT algorithm (Algorithm 1), plus the load
balance ratio R_LB.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py`` may import this module; the library never does, and this module
imports nothing from the library.

Sources (Canzona analysis page, paper-graph-ui):
* section 3.4, "Paradigm 3: Static Partitioning": a parameter belongs to the
  rank whose geometric slice of width S = |B| / R holds its first element;
* section 3.4, "The DP Load-Balance Optimization Problem": buckets are ordered
  sequences of atomic parameters with loads W(p); slicing vectors s_i cut each
  bucket at parameter boundaries; rank r's load from bucket i is the load of
  the parameters between its cuts;
* section 3.4, "The alpha-Balanced Greedy LPT Algorithm (Algorithm 1)": the
  steps implemented by ``alpha_balanced``;
* section 5, "Evaluation Methodology" (Metrics): R_LB = max_r v_r / avg_r v_r.

Readings where the pages leave a step open:
* cuts are parameter indices, non-decreasing (a rank may own no parameter of a
  bucket that has fewer parameters than there are ranks);
* the cut for rank r is searched among the boundaries at or after rank r-1's
  cut, and a tie in |Phi(u) - C| goes to the earlier boundary;
* buckets of equal load keep their original order in the LPT order;
* the Start_Index rule numbers ranks from 0 (the pages' worked example: a
  start of 1,048,577 with S = 1,048,576 falls in rank 1's slice). With
  S = |B| / R, r S <= start < (r + 1) S is start * R // |B| == r, which is
  evaluated in integers, exactly.

Every computation is a plain loop in float64 (integer sizes, float loads).
"""

from __future__ import annotations

from typing import List, Sequence, Tuple


def prefix_loads(loads: Sequence[float]) -> List[float]:
    """Phi(u) for u = 0 .. len(loads): the load of the first u parameters."""
    phi = [0.0]
    for w in loads:
        phi.append(phi[-1] + float(w))
    return phi


def static_partition(sizes: Sequence[Sequence[int]], ranks: int) -> List[List[int]]:
    """Cuts of every bucket by the Start_Index rule (no load balancing).

    Parameter p of bucket i goes to rank floor(start(p) * R / |B_i|), i.e. the
    r with r S_i <= start(p) < (r + 1) S_i for S_i = |B_i| / R, where start(p)
    is the number of elements before p in the bucket.
    Returns, per bucket, the R + 1 cut indices (rank r owns parameters
    cuts[r] .. cuts[r+1] - 1)."""
    out = []
    for bucket in sizes:
        total = sum(bucket)
        owner = []
        start = 0
        for n in bucket:
            owner.append(start * ranks // total)
            start += n
        cuts = [0] * (ranks + 1)
        for r in range(ranks + 1):
            cuts[r] = sum(1 for o in owner if o < r)
        out.append(cuts)
    return out


def alpha_balanced(loads: Sequence[Sequence[float]], ranks: int, alpha: float) -> List[List[int]]:
    """Cuts of every bucket by the alpha-Balanced Greedy LPT algorithm.

    Buckets are visited heaviest first. For bucket k: each rank's deficit
    d_r = max(0, mu - L_r) against the mean mu of all loads; the target share
    v = (1 - alpha) / R + alpha * d_r / D (the even share alone when D = 0);
    the cumulative target C grows by W^k * v_r for r = 0 .. R-2, and rank r's
    cut is the boundary whose prefix load is closest to C; rank R-1 takes the
    rest. L_r grows by the load between rank r's cuts."""
    n_buckets = len(loads)
    totals = [sum(float(w) for w in b) for b in loads]
    mu = sum(totals) / ranks
    order = sorted(range(n_buckets), key=lambda i: -totals[i])   # stable: ties keep index order
    L = [0.0] * ranks
    cuts_all: List[List[int]] = [[] for _ in range(n_buckets)]
    for k in order:
        phi = prefix_loads(loads[k])
        n = len(loads[k])
        d = [max(0.0, mu - L[r]) for r in range(ranks)]
        D = sum(d)
        if D > 0.0:
            v = [(1.0 - alpha) * (1.0 / ranks) + alpha * (d[r] / D) for r in range(ranks)]
        else:
            v = [1.0 / ranks] * ranks
        cuts = [0] * (ranks + 1)
        C = 0.0
        for r in range(ranks - 1):
            C = C + totals[k] * v[r]
            best, best_gap = cuts[r], None
            for u in range(cuts[r], n + 1):
                gap = abs(phi[u] - C)
                if best_gap is None or gap < best_gap:
                    best, best_gap = u, gap
            cuts[r + 1] = best
            L[r] += phi[cuts[r + 1]] - phi[cuts[r]]
        cuts[ranks] = n
        L[ranks - 1] += phi[n] - phi[cuts[ranks - 1]]
        cuts_all[k] = cuts
    return cuts_all


def rank_loads(loads: Sequence[Sequence[float]], cuts: Sequence[Sequence[int]], ranks: int) -> List[float]:
    """Total load of every rank over all buckets, from the cuts."""
    tot = [0.0] * ranks
    for b, c in zip(loads, cuts):
        for r in range(ranks):
            for j in range(c[r], c[r + 1]):
                tot[r] += float(b[j])
    return tot


def load_balance_ratio(values: Sequence[float]) -> float:
    """R_LB = max_r v_r / avg_r v_r."""
    return max(values) / (sum(values) / len(values))


def objectives(sizes, loads, cuts, ranks) -> Tuple[float, float]:
    """(J_DP, J_Comm): the largest deviation of a rank's total load from the
    mean, and the summed deviation of every shard's size from its bucket's
    uniform share (section 3.4, the two objectives)."""
    tot = rank_loads(loads, cuts, ranks)
    mu = sum(tot) / ranks
    j_dp = max(abs(t - mu) for t in tot)
    j_comm = 0.0
    for b, c in zip(sizes, cuts):
        share = sum(b) / ranks
        for r in range(ranks):
            j_comm += abs(sum(b[c[r]:c[r + 1]]) - share)
    return j_dp, j_comm
