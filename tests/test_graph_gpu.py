"""muon_step captured in a HIP graph (torch.cuda.graph) and replayed.

A step only launches kernels and records and waits on events. It makes no
memset, copy or host synchronisation, and it clears the work-queue counters in
its own momentum kernels. So a caller can capture it once and replay it. This
test checks that each replay leaves W, M and delta bit for bit equal to an
eager step of a second plan over a copy of the same inputs. Between replays
the program does unrelated eager work and synchronises. Bit equality is the
bar because a plan's result does not depend on addresses or on scheduling:
every tile sums its K steps in a fixed order.
"""
import time

import numpy as np
import pytest

from matrix_optimizer_step_muon_amd import muon as mu
from matrix_optimizer_step_muon_amd import workloads as wl

from gpu_helpers import log, to_device, to_host

pytestmark = pytest.mark.gpu

CASES = {
    # bf16, two chains (the default), a ragged mix with a rank-1 matrix.
    "bf16_ragged": ([(300, 700), (700, 300), (1, 5), (513, 512), (1024, 2048), (129, 1030)], "bf16"),
    # bf16, the Qwen3-1.7B layer's shapes.
    "bf16_qwen3_1p7b_layer": ([(2048, 2048), (1024, 2048), (1024, 2048), (2048, 2048), (6144, 2048),
                               (6144, 2048), (2048, 6144)], "bf16"),
    # fp32 engine, one chain: 16 matrices of 128 x 256.
    "f32_tiny": ([(128, 256)] * 16, "f32"),
    # fp32 master weights and momentum with bf16 gradients (MUON_BF16_F32_MASTER).
    "master_ragged": ([(300, 700), (700, 300), (1, 5), (1024, 2048)], "master"),
}


def _storage(dtype):
    """Storage types of (W, G, M, delta)."""
    return ("f32", "bf16", "f32", "f32") if dtype == "master" else (dtype,) * 4


def _inputs(shapes, dtype, seed):
    if dtype != "master":
        return wl.generate(wl.custom_workload(f"graph_{dtype}", shapes, dtype, seed=seed))
    return [(wl.to_storage(wl.draw(seed, i, 1, s, 0.02), "f32"), wl.to_storage(wl.draw(seed, i, 0, s, 1e-3), "bf16"),
             wl.to_storage(wl.draw(seed, i, 2, s, 1e-3), "f32")) for i, s in enumerate(shapes)]


def _device_copy(inputs, dtype):
    import torch
    sw, sg, sm, sd = _storage(dtype)
    out = []
    for (W, G, M) in inputs:
        out.append([to_device(W, sw), to_device(G, sg), to_device(M, sm),
                    torch.full(W.shape, float("nan"), dtype=torch.bfloat16 if sd == "bf16" else torch.float32,
                               device="cuda")])
    return out


def _host(dev, dtype):
    sw, _, sm, sd = _storage(dtype)
    return [(to_host(W, sw), to_host(M, sm), to_host(D, sd)) for W, _, M, D in dev]


def _median_ms(fn, n=10):
    import torch
    ts = []
    for _ in range(n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        ts.append((time.perf_counter() - t0) * 1e3)
    return sorted(ts)[n // 2]


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_equal_eager_steps(case):
    import torch
    shapes, dtype = CASES[case]
    log(f"case graph capture {case}")
    inputs = _inputs(shapes, dtype, 81)
    eager, graphed = _device_copy(inputs, dtype), _device_copy(inputs, dtype)
    plan_e, plan_g = mu.Plan(eager), mu.Plan(graphed)
    if dtype == "master":
        assert plan_g.hparams.dtype == mu.MUON_BF16_F32_MASTER
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        plan_g.step()                      # captured on `side`: nothing runs yet
    torch.cuda.synchronize()
    assert all(bool(torch.isnan(D).all()) for *_, D in graphed), "capture must not run the step"
    x = torch.randn(512, 512, device="cuda")
    for k in range(3):
        plan_e.step()
        torch.cuda.synchronize()
        g.replay()
        y = (x @ x).sum()                  # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(y)
        for i, (e, r) in enumerate(zip(_host(eager, dtype), _host(graphed, dtype))):
            for name, a, b in zip(("W", "M", "delta"), e, r):
                bad = np.count_nonzero(a.view(np.uint8) != b.view(np.uint8))
                assert bad == 0, f"{case} replay {k}: matrix {i} {shapes[i]} {name}: {bad} bytes differ"
    t_eager = _median_ms(plan_e.step)
    t_graph = _median_ms(g.replay)
    log(f"{case}: eager step {t_eager:.3f} ms, graph replay {t_graph:.3f} ms (host wall clock, synchronised)")
    del g
    plan_e.close()
    plan_g.close()


def test_graph_replays_of_the_shard_apply():
    """muon_apply (one kernel launch) captured and replayed twice equals two
    eager applies on a copy of the same shards, bit for bit."""
    import torch
    from oracle import muon_ref as ref
    log("case graph capture shard apply")
    r, c, ranks = 300, 700, 4
    W = wl.to_storage(wl.draw(82, 0, 1, (r, c), 0.02), "bf16")
    D = to_device(wl.to_storage(wl.draw(82, 0, 3, (r, c), 4e-4), "bf16"), "bf16")
    shards = ref.tp_shard_ranges(r, c, ranks, "row")
    sets = []
    for _ in range(2):
        Ps = [to_device(np.ascontiguousarray(W[rs, cs]), "bf16") for rs, cs in shards]
        sets.append((Ps, mu.ApplyPlan([(P, D[rs, cs]) for P, (rs, cs) in zip(Ps, shards)])))
    (Pe, plan_e), (Pg, plan_g) = sets
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        plan_g.apply()
    torch.cuda.synchronize()
    assert all(np.array_equal(to_host(P, "bf16"), np.ascontiguousarray(W[rs, cs])) for P, (rs, cs) in zip(Pg, shards)), \
        "capture must not run the apply"
    for k in range(2):
        plan_e.apply()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(Pe, Pg)):
            assert np.array_equal(to_host(a, "bf16"), to_host(b, "bf16")), f"replay {k}: shard {i} differs"
    del g
    plan_e.close()
    plan_g.close()
