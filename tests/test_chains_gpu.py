"""The two-chain schedule of the bf16 four-wave engine: two groups of matrices,
each with its own momentum, norm and GEMM launches on its own stream, forked at
the start of the step and joined by events. (MUON_SPLIT_PROLOGUE=0 runs one
momentum and one norm kernel over all matrices before the fork instead.)

The chains run the same tiles with the same code, so one and two chains must
give bit-identical results; and a step issued on any stream must be complete,
for work issued after it on that stream, when that work starts.
"""
import os

import numpy as np
import pytest

from matrix_optimizer_step_muon_amd import muon as mu
from matrix_optimizer_step_muon_amd import workloads as wl

from gpu_helpers import gpu_step, log, to_device, to_host

pytestmark = pytest.mark.gpu

# Several matrices of different work, so that both chains get some.
SHAPES = [(1024, 768), (768, 1536), (512, 512), (1280, 256), (300, 700), (256, 2048)]
# The schedule test adds a matrix with m in (2048, 4096] (8 x 8 blocks and the
# 4-stage update engine by default).
SCHEDULE_SHAPES = SHAPES + [(2560, 3072)]


def _with_env(name, value, fn):
    saved = os.environ.get(name)
    os.environ[name] = str(value)
    try:
        return fn()
    finally:
        if saved is None:
            del os.environ[name]
        else:
            os.environ[name] = saved


def _with_chains(n, fn):
    return _with_env("MUON_CHAINS", n, fn)


@pytest.mark.parametrize("chains,split_prologue", [(2, 1), (2, 0), (3, 1)])
def test_one_and_several_chains_agree_bitwise(chains, split_prologue):
    w = wl.custom_workload("chains", SHAPES, "bf16", seed=51)
    inputs = wl.generate(w)
    hp = w.hparams()
    log(f"case chains 1 vs {chains}, split prologue {split_prologue}")
    one = _with_chains(1, lambda: gpu_step(inputs, "bf16", hp, steps=2))
    many = _with_env("MUON_SPLIT_PROLOGUE", split_prologue,
                     lambda: _with_chains(chains, lambda: gpu_step(inputs, "bf16", hp, steps=2)))
    for i, (a, b) in enumerate(zip(one, many)):
        for name, x, y in zip(("W'", "M'", "delta"), a, b):
            assert np.array_equal(x, y), f"matrix {i} {SHAPES[i]}: {name} differs between 1 and {chains} chains"


def test_step_on_a_side_stream_is_joined():
    """A copy of W queued right after the step on the same (non-default)
    stream must see the final W, in every matrix of either chain."""
    import torch
    w = wl.custom_workload("side_stream", SHAPES, "bf16", seed=53)
    inputs = wl.generate(w)
    hp = w.hparams()
    log("case step on a side stream")
    want = _with_chains(2, lambda: gpu_step(inputs, "bf16", hp, with_delta=False))

    def run():
        dev = [[to_device(W, "bf16"), to_device(G, "bf16"), to_device(M, "bf16")] for (W, G, M) in inputs]
        plan = mu.Plan(dev, **hp)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            plan.step(side)
            copies = [d[0].clone() for d in dev]   # queued behind the step on `side`
        side.synchronize()
        out = [to_host(c, "bf16") for c in copies]
        plan.close()
        return out

    got = _with_chains(2, run)
    for i, (g, ref) in enumerate(zip(got, want)):
        assert np.array_equal(g, ref[0]), f"matrix {i} {SHAPES[i]}: W copied after the step is not the final W"


@pytest.mark.parametrize("env", [{"MUON_BLOCK": "2x8"}, {"MUON_BLOCK": "1x1", "MUON_BLOCK_ORDER": "0"},
                                 {"MUON_BLOCK_PHASES": "4x8,2x4,8x2"}, {"MUON_GEMM_VARIANT": "2"}])
def test_tile_schedule_does_not_change_results(env):
    """Block shapes and the order blocks are dealt in only move tiles between
    queues and workgroups; every tile's arithmetic is the same, so the result
    is bit for bit the default schedule's. The same holds for the engine of the
    update launches: these shapes (m <= 4096) update on the 4-stage engine by
    default, and MUON_GEMM_VARIANT=2 puts them on the 2-stage one, which sums
    the same K chunks in the same order."""
    w = wl.custom_workload("schedule", SCHEDULE_SHAPES, "bf16", seed=57)
    inputs = wl.generate(w)
    hp = w.hparams()
    log(f"case tile schedule {env}")
    ref_out = gpu_step(inputs, "bf16", hp)

    def run():
        return gpu_step(inputs, "bf16", hp)

    fn = run
    for k, v in env.items():
        fn = (lambda f, k, v: (lambda: _with_env(k, v, f)))(fn, k, v)
    got = fn()
    for i, (a, b) in enumerate(zip(ref_out, got)):
        for name, x, y in zip(("W'", "M'", "delta"), a, b):
            assert np.array_equal(x, y), f"matrix {i} {SCHEDULE_SHAPES[i]}: {name} differs under {env}"
