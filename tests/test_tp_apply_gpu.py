"""Parity of the tensor-parallel local update (muon_apply_plan / muon_apply)
with the oracle: every rank's parameter shard plus its slice of the update,
P_local + Delta W_local, over column-parallel shards (blocks of output rows)
and row-parallel shards (blocks of input columns, strided views of the update).

The kernel forms each sum in fp32 and stores it once; for two values of the
storage type that is their exactly rounded sum (pinned on the CPU in
test_oracle_pins.py), so the comparison is bit for bit.
"""
import numpy as np
import pytest

from matrix_optimizer_step_muon_amd import muon as mu
from matrix_optimizer_step_muon_amd import workloads as wl
from oracle import muon_ref as ref

from gpu_helpers import gpu_step, log, to_device, to_host

pytestmark = pytest.mark.gpu

# One Qwen3-1.7B-shaped decoder layer: q, k, v, gate and up are column-parallel
# (output rows split), o and down row-parallel (input columns split).
QWEN3_1P7B = [(2048, 2048, "column"), (1024, 2048, "column"), (1024, 2048, "column"),
              (2048, 2048, "row"), (6144, 2048, "column"), (6144, 2048, "column"),
              (2048, 6144, "row")]
# Ragged and odd cases: uneven splits, widths that are not a multiple of 4
# (the kernel's element-wise path), a single element, a tall thin matrix.
RAGGED = [(300, 700, "column"), (300, 700, "row"), (7, 13, "row"), (1, 1, "column"),
          (513, 3, "column"), (65, 130, "row")]


def _inputs(layout, dtype, seed):
    """Per matrix: W (weights, N(0, 0.02^2)) and the full update Delta W
    (N(0, (4e-4)^2), the size of lr * O entries at these widths), stored."""
    out = []
    for i, (r, c, _) in enumerate(layout):
        W = wl.to_storage(wl.draw(seed, i, 1, (r, c), 0.02), dtype)
        D = wl.to_storage(wl.draw(seed, i, 3, (r, c), 4e-4), dtype)
        out.append((W, D))
    return out


def _run_apply(layout, ranks, dtype, seed, order=None):
    """Applies every rank's shards of every matrix in one plan. Returns the
    updated P shards (host storage arrays) and the expected ones."""
    import torch
    inputs = _inputs(layout, dtype, seed)
    pairs, keys, expect = [], [], []
    keep = []
    for i, ((r, c, kind), (W, D)) in enumerate(zip(layout, inputs)):
        Dd = to_device(D, dtype)                       # the host rank's whole update
        keep.append(Dd)
        W64, D64 = wl.stored_to_f64(W, dtype), wl.stored_to_f64(D, dtype)
        for rank, (rs, cs) in enumerate(ref.tp_shard_ranges(r, c, ranks, kind)):
            if rs.stop == rs.start or cs.stop == cs.start:
                continue                               # a rank with an empty shard
            P = to_device(np.ascontiguousarray(W[rs, cs]), dtype)   # the rank's own shard
            pairs.append((P, Dd[rs, cs]))                            # a strided view for row shards
            keys.append((i, rank))
            expect.append(wl.to_storage(ref.apply_shard(W64[rs, cs], D64[rs, cs]), dtype))
    order = list(range(len(pairs))) if order is None else order
    plan = mu.ApplyPlan([pairs[k] for k in order])
    plan.apply()
    torch.cuda.synchronize()
    got = [to_host(P, dtype) for P, _ in pairs]
    plan.close()
    return got, expect, keys


def _assert_equal(got, expect, keys, label):
    for g, e, k in zip(got, expect, keys):
        bad = np.count_nonzero(g != e)
        assert bad == 0, f"{label}: matrix {k[0]} rank {k[1]}: {bad} of {g.size} elements differ"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("ranks", [2, 8])
def test_qwen3_1p7b_layer_shards(dtype, ranks):
    log(f"case tp apply qwen3-1.7B layer {dtype} TP={ranks}")
    got, expect, keys = _run_apply(QWEN3_1P7B, ranks, dtype, seed=61)
    _assert_equal(got, expect, keys, f"qwen3-1.7B {dtype} TP={ranks}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_shards(dtype):
    log(f"case tp apply ragged {dtype}")
    got, expect, keys = _run_apply(RAGGED, 3, dtype, seed=62)
    _assert_equal(got, expect, keys, f"ragged {dtype}")


def test_shard_order_does_not_matter():
    log("case tp apply reversed shard order")
    got, expect, keys = _run_apply(RAGGED, 3, "bf16", seed=63)
    n = len(got)
    got_r, _, _ = _run_apply(RAGGED, 3, "bf16", seed=63, order=list(reversed(range(n))))
    _assert_equal(got_r, expect, keys, "reversed order")


def test_apply_twice_accumulates():
    """A second apply adds the slices again (the update is in place)."""
    import torch
    log("case tp apply twice")
    layout = [(300, 700, "row")]
    (W, D), = _inputs(layout, "bf16", seed=64)
    Dd = to_device(D, "bf16")
    shards = ref.tp_shard_ranges(300, 700, 4, "row")
    Ps = [to_device(np.ascontiguousarray(W[rs, cs]), "bf16") for rs, cs in shards]
    plan = mu.ApplyPlan([(P, Dd[rs, cs]) for P, (rs, cs) in zip(Ps, shards)])
    plan.apply()
    plan.apply()
    torch.cuda.synchronize()
    W64, D64 = wl.stored_to_f64(W, "bf16"), wl.stored_to_f64(D, "bf16")
    for P, (rs, cs) in zip(Ps, shards):
        once = wl.stored_to_f64(wl.to_storage(ref.apply_shard(W64[rs, cs], D64[rs, cs]), "bf16"), "bf16")
        twice = wl.to_storage(ref.apply_shard(once, D64[rs, cs]), "bf16")
        assert np.array_equal(to_host(P, "bf16"), twice)
    plan.close()


def test_host_rank_step_then_shard_apply():
    """The lifecycle on one GPU: the host rank's step writes delta (w NULL),
    the slices of delta go to the ranks' shards of W, and each rank's shard
    becomes its W shard plus the delta slice, rounded once."""
    import torch
    log("case host-rank step then tp apply")
    w = wl.custom_workload("tp_host", [(512, 384), (256, 768)], "bf16", seed=65)
    inputs = wl.generate(w)
    hp = w.hparams()
    res = gpu_step(inputs, "bf16", hp, with_w=False)        # delta only
    for (W, _, _), (_, _, delta), (r, c), kind in zip(inputs, res, w.shapes, ["column", "row"]):
        assert delta is not None and not np.isnan(wl.stored_to_f64(delta, "bf16")).any()
        Dd = to_device(delta, "bf16")
        shards = ref.tp_shard_ranges(r, c, 4, kind)
        Ps = [to_device(np.ascontiguousarray(W[rs, cs]), "bf16") for rs, cs in shards]
        plan = mu.ApplyPlan([(P, Dd[rs, cs]) for P, (rs, cs) in zip(Ps, shards)])
        plan.apply()
        torch.cuda.synchronize()
        W64, D64 = wl.stored_to_f64(W, "bf16"), wl.stored_to_f64(delta, "bf16")
        for P, (rs, cs) in zip(Ps, shards):
            assert np.array_equal(to_host(P, "bf16"),
                                  wl.to_storage(ref.apply_shard(W64[rs, cs], D64[rs, cs]), "bf16"))
        plan.close()
