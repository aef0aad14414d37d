"""Where a parity bar comes from when it is not the stated one.

Rank-1 matrices (m = min(rows, cols) = 1) under bf16 storage. Such a matrix
has one singular value, and every Newton-Schulz iteration stores its 1 x 1
Gram and square and the row X in bf16, so each iteration perturbs that value
by up to about 2^-9 relative and the quintic passes the perturbation on to the
next iteration. Nothing averages it out across many singular values, as it
does for m >= 2. This test runs a plain bf16-storage emulation (fp64
arithmetic, every stored intermediate rounded to bf16) on random rank-1
inputs against the fp64 oracle: the relative Frobenius error of O sits around
1.8e-2 and exceeds the bf16 bar of 2e-2 for about a fifth of the inputs, but
stays below 3e-2. Rank-1 matrices are therefore held to 3e-2 in the parity
tests that draw them with fresh seeds (the bf16 path's fixed ragged case
passes 2e-2).
"""
import numpy as np

from oracle import muon_ref as ref

RANK1_BF16_BAR = 3e-2


def _bf16(x):
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _bf16_storage_ns(U, steps=5):
    a, b, c = ref.QUINTIC_COEFFS
    X = _bf16(U) / (np.linalg.norm(U) + ref.DEFAULT_EPS)
    for _ in range(steps):
        A = _bf16(X @ X.T)
        B = _bf16(b * A + c * (A @ A))
        X = _bf16(a * X + B @ X)
    return X


def test_rank_one_bf16_storage_error_is_below_its_bar():
    rng = np.random.default_rng(0)
    errs = []
    for n in (5, 64, 1000):
        for _ in range(300):
            U = rng.standard_normal((1, n))
            O = ref.orthogonalize(U, 5)
            errs.append(np.linalg.norm(_bf16_storage_ns(U) - O) / np.linalg.norm(O))
    errs = np.array(errs)
    assert 0.01 < np.median(errs) < 0.02          # the typical error is close to the bf16 bar
    assert (errs > 2e-2).mean() > 0.05            # and exceeds it for a good share of inputs
    assert errs.max() < RANK1_BF16_BAR
