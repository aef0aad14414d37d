"""muon_step_noalloc: one step in the library's static scratch, with no
allocation, against muon_plan + muon_step on copies of the same inputs.

Two calls in a row, the second on a smaller batch than the first, so the
second call runs on what the first left in the scratch. The no-allocation
step runs the same kernels over the same tiles as a plan's step (one chain;
one and two chains agree bit for bit), so the results must be equal bit for
bit, which is stricter than the parity bar. A batch too large for the
scratch is rejected before anything is enqueued.
"""

import ctypes

import numpy as np
import pytest

from gpu_helpers import compare, gpu_step, log, oracle_step, to_device, to_host
from matrix_optimizer_step_muon_amd import muon as mu
from matrix_optimizer_step_muon_amd import workloads as wl

pytestmark = pytest.mark.gpu

FIRST = [(1024, 768), (768, 1536), (300, 700), (700, 300), (1, 5), (513, 512)]
SECOND = [(640, 384), (129, 1030)]


def noalloc_step(inputs, dtype, hp):
    """One muon_step_noalloc over fresh device copies; returns (W', M', delta)."""
    import torch
    dev = []
    for (W, G, M) in inputs:
        Wd, Gd, Md = (to_device(x, dtype) for x in (W, G, M))
        Dd = torch.empty_like(Gd).fill_(float("nan"))
        dev.append([Wd, Gd, Md, Dd])
    mu.step_noalloc(dev, **hp)
    torch.cuda.synchronize()
    return [(to_host(d[0], dtype), to_host(d[2], dtype), to_host(d[3], dtype)) for d in dev]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_step_equals_planned_step_twice(dtype):
    hp_std = dict(g_std=1.0) if dtype == "f32" else {}
    for k, shapes in enumerate((FIRST, SECOND)):
        w = wl.custom_workload(f"noalloc_{dtype}_{k}", shapes, dtype, seed=91 + k, **hp_std)
        inputs = wl.generate(w)
        hp = w.hparams()
        log(f"case no-alloc {dtype} call {k + 1}: {len(shapes)} matrices")
        got = noalloc_step(inputs, dtype, hp)
        want = gpu_step(inputs, dtype, hp)
        for i, (a, b) in enumerate(zip(got, want)):
            for name, x, y in zip(("W'", "M'", "delta"), a, b):
                assert np.array_equal(x, y), f"call {k + 1} matrix {i} {shapes[i]}: {name} differs from muon_step"
        compare(got, oracle_step(inputs, dtype, hp), dtype, hp, inputs, f"no-alloc {dtype} call {k + 1}")


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    import torch
    # 4096 x 4096 bf16: X ping/pong and A, B need about 130 MiB, more than
    # the 64 MiB scratch. Rejected before any launch.
    W = torch.zeros(4096, 4096, dtype=torch.bfloat16, device="cuda")
    G = torch.randn(4096, 4096, device="cuda").mul_(1e-3).to(torch.bfloat16)
    M = torch.zeros_like(W)
    with pytest.raises(mu.MuonError) as e:
        mu.step_noalloc([(W, G, M)])
    assert e.value.status == -1 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert not torch.any(W).item() and not torch.any(M).item(), "a rejected call must not run"
