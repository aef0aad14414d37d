"""Resuming from a checkpoint, and non-finite inputs, through the C ABI.

Resume: the optimizer state of the whole-tensor step is W and the momentum
buffer M, which stay on the rank that owns the tensor (Canzona analysis page,
section 3.4, "Task abstraction as the organizing concept"). Saving them after a
step, and stepping a new plan over fresh buffers that hold the saved values,
must give exactly what a second step of the first plan gives: the plan holds
no state that carries from one step to the next.

Non-finite inputs: a NaN or an infinity in a gradient propagates, as it does
in the definition, to the whole update of that matrix (the norm and every
product mix all of its entries) and to the one momentum entry it touches; the
other matrices of the batch are untouched, bit for bit.
"""

import numpy as np
import pytest

from gpu_helpers import gpu_step, log, oracle_step
from matrix_optimizer_step_muon_amd import workloads as wl

pytestmark = pytest.mark.gpu

SHAPES = [(1024, 768), (768, 1536), (512, 512), (300, 700), (700, 300)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_resume_on_fresh_buffers_equals_two_straight_steps(dtype):
    w = wl.custom_workload(f"resume_{dtype}", SHAPES, dtype, seed=81,
                           g_std=1.0 if dtype == "f32" else 1e-3)
    inputs = wl.generate(w)
    hp = w.hparams()
    g2 = [wl.to_storage(wl.draw(82, i, 0, s, w.g_std), dtype) for i, s in enumerate(SHAPES)]
    log(f"case resume {dtype}: two straight steps")
    straight = gpu_step(inputs, dtype, hp, steps=2, grads=[None, g2])
    log(f"case resume {dtype}: one step, checkpoint W and M to the host, new plan on fresh buffers, one step")
    first = gpu_step(inputs, dtype, hp, steps=1)
    ckpt = [(W1.copy(), g2[i], M1.copy()) for i, (W1, M1, _) in enumerate(first)]
    resumed = gpu_step(ckpt, dtype, hp, steps=1)
    for i, (a, b) in enumerate(zip(straight, resumed)):
        for name, x, y in zip(("W'", "M'", "delta"), a, b):
            assert np.array_equal(x, y), f"matrix {i} {SHAPES[i]}: {name} of the resumed step differs"


@pytest.mark.parametrize("bad", [np.nan, np.inf], ids=["nan", "inf"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_non_finite_gradient_poisons_its_own_matrix_only(dtype, bad):
    w = wl.custom_workload(f"nonfinite_{dtype}", SHAPES, dtype, seed=83,
                           g_std=1.0 if dtype == "f32" else 1e-3)
    inputs = wl.generate(w)
    hp = w.hparams()
    hit, at = 4, (5, 7)   # the tall 700 x 300 matrix
    G = wl.stored_to_f64(inputs[hit][1], dtype).astype(np.float32)
    G[at] = bad
    poisoned = list(inputs)
    poisoned[hit] = (inputs[hit][0], wl.to_storage(G, dtype), inputs[hit][2])
    log(f"case non-finite gradient {dtype} {bad}")
    clean = gpu_step(inputs, dtype, hp)
    got = gpu_step(poisoned, dtype, hp)

    # The definition: every entry of O and W' of the poisoned matrix is NaN.
    with np.errstate(invalid="ignore", over="ignore"):
        _, Mr, Or = oracle_step([poisoned[hit]], dtype, hp)[0]
    assert np.isnan(Or).all(), "the oracle's O should be NaN everywhere"

    Wg, Mg, Dg = (wl.stored_to_f64(x, dtype) for x in got[hit])
    assert np.isnan(Dg).all(), "delta of the poisoned matrix must be NaN everywhere"
    assert np.isnan(Wg).all(), "W' of the poisoned matrix must be NaN everywhere"
    mask = np.zeros(Mg.shape, bool)
    mask[at] = True
    if np.isnan(bad):
        assert np.isnan(Mg[at])
    else:
        assert Mg[at] == Mr[at] == np.inf
    assert np.array_equal(got[hit][1][~mask], clean[hit][1][~mask]), "M' changed away from the poisoned entry"
    for i in range(len(SHAPES)):
        if i == hit:
            continue
        for name, x, y in zip(("W'", "M'", "delta"), clean[i], got[i]):
            assert np.array_equal(x, y), f"matrix {i} {SHAPES[i]}: {name} changed by another matrix's NaN"
