"""The library's DP static partition (muon_dp_partition, muon_dp_partition_static:
host code, no GPU) against the oracle in oracle/partition_ref.py, cut for cut,
on random instances and on a Qwen3-32B-shaped parameter buffer."""
import math
import random

import pytest

from matrix_optimizer_step_muon_amd import muon as mu
from oracle import muon_ref as ref
from oracle import partition_ref as pr


def _random_instance(rng):
    R = rng.choice([1, 2, 3, 5, 8, 32, 128])
    buckets = [[rng.randint(1, 10 ** rng.randint(0, 8)) for _ in range(rng.randint(1, 40))]
               for _ in range(rng.randint(1, 30))]
    return R, buckets


def test_static_rule_worked_example():
    """The pages' Start_Index example (Canzona analysis page, section 3.4,
    Paradigm 3) through the library: with stride S = 1,048,576, the parameter
    starting at element 1,048,577 belongs to rank 1."""
    S = 1_048_576
    cuts, _ = mu.dp_partition([[S + 1, S, 2 * S - 1]], 4, alpha=None)
    assert cuts == [[0, 1, 2, 3, 3]]


@pytest.mark.parametrize("seed", range(60))
def test_static_rule_matches_the_oracle(seed):
    rng = random.Random(seed)
    R, buckets = _random_instance(rng)
    cuts, loads = mu.dp_partition(buckets, R, alpha=None)
    assert cuts == pr.static_partition(buckets, R)
    assert loads == pr.rank_loads(buckets, cuts, R)


@pytest.mark.parametrize("seed", range(60))
@pytest.mark.parametrize("alpha", [0.0, 0.25, 1.0])
def test_alpha_balanced_matches_the_oracle(seed, alpha):
    rng = random.Random(1000 + seed)
    R, buckets = _random_instance(rng)
    cuts, loads = mu.dp_partition(buckets, R, alpha=alpha)
    assert cuts == pr.alpha_balanced(buckets, R, alpha)
    assert loads == pr.rank_loads(buckets, cuts, R)


@pytest.mark.parametrize("seed", range(30))
def test_float_loads_and_ties_match_the_oracle(seed):
    """Loads other than the sizes (a FLOP cost), and buckets built to tie:
    equal loads, zero loads, repeated buckets."""
    rng = random.Random(2000 + seed)
    R = rng.choice([2, 3, 4, 7])
    sizes = [[rng.choice([1, 2, 4]) for _ in range(rng.randint(1, 9))] for _ in range(rng.randint(1, 8))]
    sizes += [list(b) for b in sizes[: rng.randint(0, len(sizes))]]
    loads = [[rng.choice([0.0, 0.5, 1.0, 2.0, 1.5e9]) for _ in b] for b in sizes]
    for alpha in (0.0, 0.5, 1.0):
        cuts, rl = mu.dp_partition(sizes, R, alpha=alpha, loads=loads)
        assert cuts == pr.alpha_balanced(loads, R, alpha)
        assert rl == pr.rank_loads(loads, cuts, R)
    cuts, rl = mu.dp_partition(sizes, R, alpha=None, loads=loads)
    assert cuts == pr.static_partition(sizes, R)
    assert rl == pr.rank_loads(loads, cuts, R)


def qwen3_32b_buffer(tp=1):
    """Sizes and Muon FLOP loads (vectors: their element count) of the
    Qwen3-32B-shaped buffer of the workloads module."""
    from matrix_optimizer_step_muon_amd import workloads as wl
    buckets = wl.qwen3_32b_param_buffer(tp=tp)
    sizes = [[math.prod(p) for p in b] for b in buckets]
    flops = [[float(ref.step_flops(*p)) if len(p) == 2 else float(math.prod(p)) for p in b] for b in buckets]
    return sizes, flops


@pytest.mark.parametrize("tp", [1, 8])
def test_qwen3_32b_buffer_at_dp32(tp):
    sizes, flops = qwen3_32b_buffer(tp)
    R = 32
    for alpha in (None, 0.0, 0.5, 1.0):
        for loads in (None, flops):
            cuts, rl = mu.dp_partition(sizes, R, alpha=alpha, loads=loads)
            want = (pr.static_partition(sizes, R) if alpha is None
                    else pr.alpha_balanced(loads if loads else sizes, R, alpha))
            assert cuts == want
    # balancing by numel flattens the per-rank memory (the pages' motivation)
    static_mem = pr.load_balance_ratio(mu.dp_partition(sizes, R, alpha=None)[1])
    balanced_mem = pr.load_balance_ratio(mu.dp_partition(sizes, R, alpha=1.0)[1])
    assert balanced_mem < static_mem


def test_validation():
    with pytest.raises(mu.MuonError, match="alpha"):
        mu.dp_partition([[1, 2]], 2, alpha=1.5)
    with pytest.raises(mu.MuonError, match="ranks"):
        mu.dp_partition([[1, 2]], 0)
    with pytest.raises(mu.MuonError, match="bucket"):
        mu.dp_partition([[1, 2], []], 2)
    with pytest.raises(mu.MuonError, match="sizes"):
        mu.dp_partition([[1, 0]], 2)
    with pytest.raises(mu.MuonError, match="loads"):
        mu.dp_partition([[1, 2]], 2, loads=[[1.0, -1.0]])
    with pytest.raises(mu.MuonError, match="loads"):
        mu.dp_partition([[1, 2]], 2, loads=[[1.0, float("nan")]])
