"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bars: relative Frobenius error <= 1e-4 for the fp32 path and <= 2e-2 for the
bf16 path, checked on:
- O, recovered from the delta output;
- the momentum buffer M';
- the weights W'.
Sizes span several tiles and ragged tails. The full-size cases run the
Qwen3-32B layer, the 28 Qwen3-1.7B layers and the Qwen3-32B rank share in the
plan and launch configuration that bench.py times: every matrix of the
Qwen3-32B layer, and one or more of every shape of the other two, are compared
with the oracle in full, and properties that hold at any size are checked on
every matrix.
"""

import functools

import numpy as np
import pytest

from gpu_helpers import TOL, compare, gpu_step, log, oracle_step
from matrix_optimizer_step_muon_amd import workloads as wl
from oracle import muon_ref as ref

pytestmark = pytest.mark.gpu


def run_case(wload, label, steps=1, **kw):
    inputs = wl.generate(wload)
    hp = wload.hparams()
    log(f"case {label}: {len(inputs)} matrices, dtype {wload.dtype}, hp {hp}")
    gpu = gpu_step(inputs, wload.dtype, hp, steps=steps, **kw)
    want = oracle_step(inputs, wload.dtype, hp, steps=steps)
    return compare(gpu, want, wload.dtype, hp, inputs, label)


def test_tiny_f32_batch():
    run_case(wl.WORKLOADS["tiny_f32_16x128x256"], "tiny_f32_16x128x256")


def test_qwen3_1p7b_layer_bf16():
    run_case(wl.WORKLOADS["qwen3_1p7b_layer"], "qwen3_1p7b_layer")


RAGGED = [(1000, 3000), (3000, 1000), (1, 5), (5, 1), (1, 1), (256, 256), (300, 700),
          (700, 300), (513, 512), (129, 1030), (64, 2048)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_heterogeneous_batch(dtype):
    w = wl.custom_workload(f"ragged_{dtype}", RAGGED, dtype, seed=21,
                           g_std=1.0 if dtype == "f32" else 1e-3, w_std=0.02)
    run_case(w, f"ragged_{dtype}")


@pytest.mark.parametrize("ns_steps", [0, 1, 2])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ns_step_counts(dtype, ns_steps):
    w = wl.custom_workload(f"steps{ns_steps}_{dtype}", [(384, 640), (640, 384), (200, 200)], dtype,
                           seed=31, ns_steps=ns_steps)
    run_case(w, f"ns_steps={ns_steps} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_without_nesterov(dtype):
    w = wl.custom_workload(f"plain_{dtype}", [(512, 768), (768, 512)], dtype, seed=41, nesterov=False)
    run_case(w, f"nesterov=False {dtype}")


@pytest.mark.parametrize("coeffs", [(1.5, -0.5, 0.0), (2.0, -1.5, 0.5)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_other_polynomial_coefficients(dtype, coeffs):
    """The step for any (a, b, c). c = 0 is the cubic iteration, where B = b*A
    needs no product; c != 0 folds b*A into the A*A product."""
    w = wl.custom_workload(f"coeffs_{dtype}", [(384, 640), (640, 384), (300, 300)], dtype,
                           seed=35, ns_steps=4)
    inputs = wl.generate(w)
    hp = dict(w.hparams(), coeffs=coeffs)
    log(f"case coeffs={coeffs} {dtype}")
    gpu = gpu_step(inputs, dtype, hp)
    want = oracle_step(inputs, dtype, hp)
    compare(gpu, want, dtype, hp, inputs, f"coeffs={coeffs} {dtype}")


SPLIT_SHAPES = [(1000, 3000), (3000, 1000), (300, 2300), (129, 1030), (1, 5), (512, 4096)]


def _with_env(env, fn):
    import os
    saved = {k: os.environ.get(k) for k in env}
    os.environ.update({k: str(v) for k, v in env.items()})
    try:
        return fn()
    finally:
        for k, v in saved.items():
            if v is None:
                del os.environ[k]
            else:
                os.environ[k] = v


@pytest.mark.parametrize("split", [2, 3, 5])
def test_split_k_gram_pieces(split):
    """MUON_SPLIT_K=S cuts every Gram tile into min(S, K/512) pieces along K
    (uneven ones too: 9 chunks of 256 in 4 pieces, say), whose fp32 partial
    sums a reduce launch adds in piece order. The step still meets the bar
    against the oracle, it is deterministic, and one and two chains (the
    pieces of a matrix do not depend on the chains) agree bit for bit."""
    w = wl.custom_workload(f"split{split}", SPLIT_SHAPES, "bf16", seed=23)
    inputs = wl.generate(w)
    hp = w.hparams()
    log(f"case split-K {split}")
    got = _with_env({"MUON_SPLIT_K": split}, lambda: gpu_step(inputs, "bf16", hp, steps=2))
    want = oracle_step(inputs, "bf16", hp, steps=2)
    compare(got, want, "bf16", hp, inputs, f"split-K {split}")
    again = _with_env({"MUON_SPLIT_K": split}, lambda: gpu_step(inputs, "bf16", hp, steps=2))
    one = _with_env({"MUON_SPLIT_K": split, "MUON_CHAINS": 1}, lambda: gpu_step(inputs, "bf16", hp, steps=2))
    for i in range(len(SPLIT_SHAPES)):
        for name, x, y, z in zip(("W'", "M'", "delta"), got[i], again[i], one[i]):
            assert np.array_equal(x, y), f"matrix {i}: {name} differs between two split runs"
            assert np.array_equal(x, z), f"matrix {i}: {name} differs between one and two chains"


def test_bf16_stores_round_to_nearest_even():
    """M' = beta*M + G is formed in fp32 and stored once as bf16. Every stored
    value must be the nearest-even bf16 of the fp32 value, whether the fp32
    value was formed with one rounding (fused) or two."""
    shapes = [(512, 768), (333, 200)]
    w = wl.custom_workload("rne", shapes, "bf16", seed=37, ns_steps=0, g_std=1.0)
    inputs = wl.generate(w)
    gpu = gpu_step(inputs, "bf16", w.hparams())
    beta = np.float32(w.beta)
    for (Wg, Mg, Dg), (W, G, M) in zip(gpu, inputs):
        g = wl.bf16_bits_to_f32(G)
        m = wl.bf16_bits_to_f32(M)
        fused = (beta.astype(np.float64) * m.astype(np.float64) + g.astype(np.float64)).astype(np.float32)
        split = (beta * m + g).astype(np.float32)
        ok = (Mg == wl.f32_to_bf16_bits(fused)) | (Mg == wl.f32_to_bf16_bits(split))
        assert ok.all(), f"{int((~ok).sum())} of {ok.size} M' values are not RNE of beta*M + G"


def test_zero_gradient_and_momentum_give_zero_update():
    shapes = [(300, 500), (500, 300)]
    inputs = [(wl.to_storage(wl.draw(5, i, 1, s, 0.02), "bf16"),
               wl.to_storage(np.zeros(s, np.float32), "bf16"),
               wl.to_storage(np.zeros(s, np.float32), "bf16")) for i, s in enumerate(shapes)]
    gpu = gpu_step(inputs, "bf16", dict(lr=0.02, beta=0.95))
    for (Wg, Mg, Dg), (W, _, _) in zip(gpu, inputs):
        np.testing.assert_array_equal(Wg, W)
        assert not np.any(wl.stored_to_f64(Dg, "bf16")), "delta must be exactly zero"
        assert not np.any(wl.stored_to_f64(Mg, "bf16"))


def test_two_consecutive_steps_carry_momentum():
    w = wl.custom_workload("two_steps", [(512, 1024), (1024, 512)], "bf16", seed=51)
    inputs = wl.generate(w)
    g2 = [wl.to_storage(wl.draw(99, i, 0, s, 1e-3), "bf16") for i, s in enumerate(w.shapes)]
    grads = [None, g2]
    hp = w.hparams()
    gpu = gpu_step(inputs, "bf16", hp, steps=2, grads=grads)
    want = oracle_step(inputs, "bf16", hp, steps=2, grads=grads)
    compare(gpu, want, "bf16", hp, inputs, "two steps")


def test_result_is_independent_of_descriptor_order_and_deterministic():
    w = wl.custom_workload("order", [(256, 768), (768, 256), (512, 512), (100, 900)], "bf16", seed=61)
    inputs = wl.generate(w)
    hp = w.hparams()
    a = gpu_step(inputs, "bf16", hp)
    b = gpu_step(inputs, "bf16", hp, order=[3, 1, 0, 2])
    c = gpu_step(inputs, "bf16", hp)
    for x, y, z in zip(a, b, c):
        for u, v, t in zip(x, y, z):
            np.testing.assert_array_equal(u, v)
            np.testing.assert_array_equal(u, t)


def test_delta_only_mode_leaves_no_weight_write():
    w = wl.custom_workload("delta_only", [(640, 384)], "bf16", seed=71)
    inputs = wl.generate(w)
    hp = w.hparams()
    gpu = gpu_step(inputs, "bf16", hp, with_w=False)
    want = oracle_step(inputs, "bf16", hp)
    compare(gpu, want, "bf16", hp, inputs, "delta only")


# Full-size workloads, in the plan and launch configuration bench.py times.
# Each workload's HIP step runs once (the first case that needs it) and its
# outputs are kept while that workload's cases run; every listed matrix is then
# compared with the oracle in full, one case per matrix, so that no case runs
# for long. Per workload:
# - the Qwen3-32B layer: all seven matrices (q, k, v, o, gate, up, down);
# - the 28 Qwen3-1.7B layers: one matrix of each of the seven shapes, taken
#   from seven different layers;
# - the Qwen3-32B rank share: layer 1's q, o and down, the two extra
#   1024 x 5120 matrices and the extra 25600 x 5120 one.
# A last case per workload checks properties that hold at any size on every
# matrix of the batch.
FULL_ORACLE = {
    "qwen3_32b_layer": list(range(7)),
    "qwen3_1p7b_28_layers": [0, 7 * 5 + 1, 7 * 10 + 2, 7 * 14 + 3, 7 * 19 + 4, 7 * 23 + 5, 7 * 27 + 6],
    "qwen3_32b_rank_share": [7, 10, 13, 14, 15, 16],
}
FULL_CASES = [(name, i) for name, idx in FULL_ORACLE.items() for i in idx + [None]]


@functools.lru_cache(maxsize=1)
def _full_run(name):
    """(inputs, HIP outputs) of one full-size workload; one workload is held
    at a time."""
    wload = wl.WORKLOADS[name]
    log(f"case {name}: generating inputs ({len(wload.shapes)} matrices, {wload.numel / 1e6:.0f} M elements)")
    inputs = wl.generate(wload)
    log(f"case {name}: running the HIP step")
    gpu = gpu_step(inputs, "bf16", wload.hparams())
    return inputs, gpu


def _full_size_properties(name, inputs, gpu, hp):
    """On every matrix of the batch:
    - M' on 20000 sampled elements against the elementwise definition;
    - W' against W + delta everywhere (each is rounded once from one fp32
      update);
    - the singular values of O within the quintic's reachable interval after
      five steps. Square Gaussian matrices have smallest singular values near
      0, which five steps do not lift into the band, so for them only the
      upper bound is checked."""
    import torch
    rng = np.random.default_rng(0)
    lo, top = 0.681831, 1.202369
    for i, ((W, G, M), (Wg, Mg, Dg)) in enumerate(zip(inputs, gpu)):
        r, c = W.shape
        idx = rng.integers(0, r * c, 20000)
        m_ref = 0.95 * wl.stored_to_f64(M.reshape(-1)[idx], "bf16") + wl.stored_to_f64(G.reshape(-1)[idx], "bf16")
        assert wl.rel_fro(wl.stored_to_f64(Mg.reshape(-1)[idx], "bf16"), m_ref) < 4e-3
        # W' and delta are each rounded once to bf16 from the same fp32 update,
        # so W' - (W + delta) is within half an ulp of W' plus half an ulp of delta.
        Wf, Wgf, Df = (wl.stored_to_f64(x, "bf16") for x in (W, Wg, Dg))
        assert np.all(np.abs(Wgf - (Wf + Df)) <= (np.abs(Wgf) + np.abs(Df)) * 2.0 ** -8 + 1e-30)
        O = torch.from_numpy(-Df / (hp["lr"] * ref.update_scale(r, c))).cuda().float()
        O = O if r <= c else O.T
        ev = torch.linalg.eigvalsh((O @ O.T).double()).cpu().numpy()
        sv = np.sqrt(np.clip(ev, 0, None))
        if i < 8 or i % 16 == 0:
            log(f"{name} matrix {i} {r}x{c}: singular values of O in [{sv.min():.4f}, {sv.max():.4f}]")
        assert sv.max() < top * 1.03, f"{name} matrix {i}: sigma_max {sv.max()}"
        if r != c:
            assert sv.min() > lo * 0.97, f"{name} matrix {i} ({r}x{c}): sigma_min {sv.min()}"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,index", FULL_CASES,
                         ids=[f"{n}-{'properties' if i is None else i}" for n, i in FULL_CASES])
def test_full_size_against_oracle(name, index):
    """One matrix of a full-size workload against the oracle on O, M' and W'
    (index None: the properties above, on every matrix)."""
    wload = wl.WORKLOADS[name]
    hp = wload.hparams()
    inputs, gpu = _full_run(name)
    if index is None:
        _full_size_properties(name, inputs, gpu, hp)
        return
    r, c = wload.shapes[index]
    log(f"case {name}: oracle on matrix {index} ({r}x{c})")
    want = oracle_step([inputs[index]], "bf16", hp)
    compare([gpu[index]], want, "bf16", hp, [inputs[index]], f"{name} full size #{index}", full_size=True)
