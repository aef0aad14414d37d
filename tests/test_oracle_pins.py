"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

The pages print no numeric Muon example, so the oracle is pinned by:
- closed forms: the SVD form of the odd-polynomial iteration, and the
  semi-orthogonal and rank-1 cases;
- the scalar dynamics of the quintic: its attracting band and the thresholds
  into it;
- convergence of the cubic iteration to the polar factor;
- invariances: transpose and scale;
- brute-force loops on tiny inputs;
- the degenerate cases.
Each test says which plausible oracle mistake would make it fail.
"""

import math

import numpy as np
import pytest

from oracle import muon_ref as ref

A, B, C = ref.QUINTIC_COEFFS


def p(x, coeffs=ref.QUINTIC_COEFFS):
    a, b, c = coeffs
    return a * x + b * x ** 3 + c * x ** 5


def p_iter(x, n, coeffs=ref.QUINTIC_COEFFS):
    for _ in range(n):
        x = p(x, coeffs)
    return x


def svd_closed_form(U, steps, coeffs=ref.QUINTIC_COEFFS, eps=ref.DEFAULT_EPS):
    """Spectral form of the fixed-count odd-polynomial iteration: the singular
    vectors of U are kept, and every normalised singular value goes through
    p, T times."""
    Us, s, Vt = np.linalg.svd(U, full_matrices=False)
    norm = math.sqrt(float(np.sum(s ** 2)))
    s0 = s / (norm + eps)
    return (Us * p_iter(s0, steps, coeffs)) @ Vt


def relerr(x, y):
    return np.linalg.norm(x - y) / np.linalg.norm(y)


# ------------------------------------------------------------------ P-1 momentum

def test_scalar_momentum_nesterov():
    # beta = 0.95, M = 1, G = 2: M' = 0.95 + 2 = 2.95, U = 2 + 0.95 * 2.95 = 4.8025.
    # The EMA form, (1 - beta) * G, would give M' = 1.05. The look-ahead on the
    # old buffer would give U = 2.95.
    M_new, U = ref.momentum_update(np.array([[2.0]]), np.array([[1.0]]), 0.95, True)
    assert M_new[0, 0] == pytest.approx(2.95, abs=1e-15)
    assert U[0, 0] == pytest.approx(4.8025, abs=1e-15)
    M_new, U = ref.momentum_update(np.array([[2.0]]), np.array([[1.0]]), 0.95, False)
    assert U[0, 0] == pytest.approx(2.95, abs=1e-15)


def test_momentum_returned_by_step_is_elementwise():
    rng = np.random.default_rng(11)
    W, G, M = (rng.standard_normal((3, 4)) for _ in range(3))
    _, M_new, _ = ref.muon_step(W, G, M, lr=0.02, beta=0.9)
    for i in range(3):
        for j in range(4):
            assert M_new[i, j] == pytest.approx(0.9 * M[i, j] + G[i, j], abs=1e-15)


# ----------------------------------------------------------------- P-2 / P-3

def test_frobenius_norm_brute_force():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((5, 7))
    acc = 0.0
    for i in range(5):
        for j in range(7):
            acc += X[i, j] * X[i, j]
    assert ref.frobenius_norm(X) == pytest.approx(math.sqrt(acc), rel=1e-15)


def _loop_matmul(X, Y):
    n, k = X.shape
    k2, m = Y.shape
    assert k == k2
    Z = np.zeros((n, m))
    for i in range(n):
        for j in range(m):
            s = 0.0
            for t in range(k):
                s += X[i, t] * Y[t, j]
            Z[i, j] = s
    return Z


@pytest.mark.parametrize("shape", [(3, 5, 4), (4, 7, 4)])
def test_matmul_brute_force(shape):
    n, k, m = shape
    rng = np.random.default_rng(2)
    X, Y = rng.standard_normal((n, k)), rng.standard_normal((k, m))
    np.testing.assert_allclose(X @ Y, _loop_matmul(X, Y), rtol=1e-13, atol=1e-13)


def test_one_ns_step_brute_force():
    # One iteration computed entry by entry with loops, from the definition
    # X' = a X + (b X X^T + c (X X^T)^2) X. It pins the order of the products:
    # X^T X in place of X X^T, or X B in place of B X, both fail here.
    rng = np.random.default_rng(3)
    X = rng.standard_normal((3, 5)) * 0.2
    Xt = X.T.copy()
    Am = _loop_matmul(X, Xt)
    A2 = _loop_matmul(Am, Am)
    Bm = np.zeros((3, 3))
    for i in range(3):
        for j in range(3):
            Bm[i, j] = B * Am[i, j] + C * A2[i, j]
    BX = _loop_matmul(Bm, X)
    want = np.zeros_like(X)
    for i in range(3):
        for j in range(5):
            want[i, j] = A * X[i, j] + BX[i, j]
    np.testing.assert_allclose(ref.newton_schulz(X, 1), want, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------- P-4 SVD closed form

@pytest.mark.parametrize("shape", [(8, 16), (16, 8), (12, 12), (1, 5), (5, 1), (3, 40)])
@pytest.mark.parametrize("steps", [0, 1, 2, 5])
def test_orthogonalize_matches_svd_closed_form(shape, steps):
    rng = np.random.default_rng(hash((shape, steps)) % 2**32)
    U = rng.standard_normal(shape)
    got = ref.orthogonalize(U, steps)
    np.testing.assert_allclose(got, svd_closed_form(U, steps), rtol=0, atol=1e-10 * np.abs(got).max())
    assert relerr(got, svd_closed_form(U, steps)) < 1e-10


def test_eps_sits_beside_the_norm():
    # With ||U|| = eps the first iterate is U / (2 eps). The variant
    # sqrt(||U||^2 + eps) would give a very different scale, and this case
    # would catch it.
    rng = np.random.default_rng(5)
    U = rng.standard_normal((4, 9))
    U *= ref.DEFAULT_EPS / np.linalg.norm(U)
    np.testing.assert_allclose(ref.orthogonalize(U, 0), U / (2 * ref.DEFAULT_EPS), rtol=1e-12)
    got = ref.orthogonalize(U, 5)
    assert relerr(got, svd_closed_form(U, 5)) < 1e-10


def test_full_step_matches_closed_form_through_momentum():
    rng = np.random.default_rng(6)
    W, G, M = (rng.standard_normal((10, 6)) for _ in range(3))
    W_new, M_new, O = ref.muon_step(W, G, M, lr=0.02, beta=0.95)
    U = G + 0.95 * (0.95 * M + G)
    np.testing.assert_allclose(O, svd_closed_form(U, 5), rtol=0, atol=1e-11)
    np.testing.assert_allclose(W_new, W - 0.02 * math.sqrt(10 / 6) * svd_closed_form(U, 5),
                               rtol=0, atol=1e-12)


# ------------------------------------------------------------- P-5 quintic band

def _band():
    """Critical points of p from p'(x) = a + 3b x^2 + 5c x^4 = 0, solved as a
    quadratic in x^2. The band is [p(x_min), p(p(x_min))], where x_min is the
    local minimum."""
    disc = math.sqrt(9 * B * B - 20 * A * C)
    x_max = math.sqrt((-3 * B - disc) / (10 * C))
    x_min = math.sqrt((-3 * B + disc) / (10 * C))
    lo = p(x_min)
    return x_max, x_min, lo, p(lo)


def test_quintic_band_values():
    x_max, x_min, lo, hi = _band()
    assert x_max == pytest.approx(0.554529, abs=1e-6)
    assert p(x_max) == pytest.approx(1.202369, abs=1e-6)
    assert x_min == pytest.approx(1.050136, abs=1e-6)
    assert lo == pytest.approx(0.681831, abs=1e-6)
    assert hi == pytest.approx(1.134357, abs=1e-6)
    # The band maps into itself.
    xs = np.linspace(lo, hi, 20001)
    assert p(xs).min() >= lo - 1e-12 and p(xs).max() <= hi + 1e-12
    # After k steps, every x in [t_k, 1] lands in the band. The thresholds are
    # found by bisection: p(t_k) = t_{k-1}, with t_0 = lo.
    ts = [lo]
    for _ in range(5):
        l, r = 0.0, x_max
        for _ in range(200):
            mid = 0.5 * (l + r)
            l, r = (mid, r) if p(mid) < ts[-1] else (l, mid)
        ts.append(l)
    assert ts[1] == pytest.approx(0.210663, abs=1e-6)
    assert ts[4] == pytest.approx(0.005184, abs=1e-6)
    assert ts[5] == pytest.approx(0.001505, abs=1e-6)
    # [lo, hi] maps into itself. After a fixed count of steps, though, a value
    # that sits at the local maximum x_max on the last step ends at
    # p(x_max) = 1.2024 > hi. So the set reachable from [t_k, 1] in k steps is
    # [lo, p(x_max)].
    top = p(x_max)
    for k in (4, 5):
        ys = p_iter(np.linspace(ts[k] * (1 + 1e-9), 1.0, 200001), k)
        assert ys.min() >= lo - 1e-9 and ys.max() <= top + 1e-9
        assert ys.max() > hi
    # Just below t_5, five steps fall short of the band.
    assert p_iter(ts[5] * 0.99, 5) < lo


@pytest.mark.parametrize("shape", [(8, 32), (32, 8), (6, 50)])
def test_output_singular_values_in_band(shape):
    x_max, _, lo, hi = _band()
    rng = np.random.default_rng(7)
    U = rng.standard_normal(shape)
    s0 = np.linalg.svd(U, compute_uv=False) / np.linalg.norm(U)
    assert s0.min() > 0.0016         # above t_5, so five steps reach the band
    s = np.linalg.svd(ref.orthogonalize(U, 5), compute_uv=False)
    assert s.min() >= lo - 1e-9 and s.max() <= p(x_max) + 1e-9
    # One more step from there stays in the invariant band [lo, hi].
    s6 = np.linalg.svd(ref.orthogonalize(U, 6), compute_uv=False)
    assert s6.min() >= lo - 1e-9 and s6.max() <= hi + 1e-9
    # Same singular subspaces as the input.
    O = ref.orthogonalize(U, 5)
    Us, _, Vt = np.linalg.svd(U, full_matrices=False)
    core = Us.T @ O @ Vt.T
    np.testing.assert_allclose(core, np.diag(np.diag(core)), atol=1e-10)


# ------------------------------------------------- P-6 cubic NS -> polar factor

def test_cubic_newton_schulz_converges_to_polar_factor():
    rng = np.random.default_rng(8)
    for shape in [(6, 9), (9, 6), (7, 7)]:
        U = rng.standard_normal(shape)
        Us, _, Vt = np.linalg.svd(U, full_matrices=False)
        O = ref.orthogonalize(U, 100, coeffs=(1.5, -0.5, 0.0))
        assert relerr(O, Us @ Vt) < 1e-10


# ---------------------------------------------------------- P-7 / P-8 invariances

@pytest.mark.parametrize("shape", [(7, 11), (9, 9), (11, 7)])
def test_transpose_equivariance(shape):
    rng = np.random.default_rng(9)
    U = rng.standard_normal(shape)
    assert relerr(ref.orthogonalize(U.T), ref.orthogonalize(U).T) < 1e-12


@pytest.mark.parametrize("kappa", [1e-3, 1e3])
def test_scale_invariance(kappa):
    rng = np.random.default_rng(10)
    U = rng.standard_normal((6, 13))
    got = ref.orthogonalize(kappa * U, 5, eps=kappa * ref.DEFAULT_EPS)
    assert relerr(got, ref.orthogonalize(U, 5)) < 1e-12
    # With the fixed eps the change is of order eps / ||kappa U||.
    assert relerr(ref.orthogonalize(kappa * U, 5), ref.orthogonalize(U, 5)) < 1e-4


# ------------------------------------------------ P-9 semi-orthogonal closed form

@pytest.mark.parametrize("r,c", [(24, 6), (16, 16), (6, 24), (64, 16)])
def test_semi_orthogonal_closed_form(r, c):
    rng = np.random.default_rng(12)
    Q, _ = np.linalg.qr(rng.standard_normal((max(r, c), min(r, c))))
    Q = Q if r >= c else Q.T                     # r x c with orthonormal short side
    beta, lr = 0.95, 0.02
    G = Q / (1 + beta)                           # zero momentum: U = (1 + beta) G = Q
    W_new, M_new, O = ref.muon_step(np.zeros((r, c)), G, np.zeros((r, c)), lr=lr, beta=beta)
    k = min(r, c)
    sigma = p_iter(1.0 / (math.sqrt(k) + ref.DEFAULT_EPS), 5)
    np.testing.assert_allclose(O, sigma * Q, rtol=0, atol=1e-12)
    scale = math.sqrt(r / c) if r > c else 1.0
    np.testing.assert_allclose(W_new, -lr * scale * sigma * Q, rtol=0, atol=1e-12)
    np.testing.assert_allclose(M_new, G, rtol=0, atol=0)


def test_semi_orthogonal_value_1_over_4():
    assert p_iter(0.25, 5) == pytest.approx(0.714526261, abs=1e-9)


# ------------------------------------------------------------------- P-10 rank 1

def test_rank_one_closed_form():
    rng = np.random.default_rng(13)
    u, v = rng.standard_normal(9), rng.standard_normal(5)
    U = np.outer(u, v)
    nu = np.linalg.norm(U)
    O = ref.orthogonalize(U, 5)
    s0 = nu / (nu + ref.DEFAULT_EPS)
    want = p_iter(s0, 5) * np.outer(u, v) / (np.linalg.norm(u) * np.linalg.norm(v))
    assert relerr(O, want) < 1e-9
    assert A + B + C == pytest.approx(0.701, abs=1e-12)
    assert p_iter(1.0, 5) == pytest.approx(0.696436409, abs=1e-9)


# ------------------------------------------------------ P-11 / P-12 degenerate

def test_zero_steps_is_normalisation():
    rng = np.random.default_rng(14)
    U = rng.standard_normal((5, 8))
    np.testing.assert_allclose(ref.orthogonalize(U, 0),
                               U / (np.linalg.norm(U) + ref.DEFAULT_EPS), rtol=1e-15)


def test_zero_input_gives_zero_update():
    W = np.arange(12.0).reshape(3, 4)
    W_new, M_new, O = ref.muon_step(W, np.zeros((3, 4)), np.zeros((3, 4)), lr=0.02, beta=0.95)
    assert np.all(O == 0) and np.all(W_new == W) and np.all(M_new == 0)
    assert not np.isnan(O).any()


def test_nan_propagates():
    G = np.ones((3, 4))
    G[1, 2] = np.nan
    W_new, _, _ = ref.muon_step(np.zeros((3, 4)), G, np.zeros((3, 4)), lr=0.02, beta=0.95)
    assert np.isnan(W_new).all()


def test_update_scale_orientation():
    # Rows and columns are the (out, in) shape of the weight as stored.
    assert ref.update_scale(25600, 5120) == pytest.approx(math.sqrt(5))
    assert ref.update_scale(5120, 25600) == 1.0
    assert ref.update_scale(8192, 5120) == pytest.approx(math.sqrt(1.6))


# ------------------------------------------------------------------ flop count

@pytest.mark.parametrize("r,c", [(1, 1), (3, 5), (5, 3), (4, 4)])
def test_step_flops_brute_force_count(r, c):
    m, n = min(r, c), max(r, c)
    per_iter = 0
    for i in range(m):
        for j in range(i, m):
            per_iter += 2 * n          # one entry of the symmetric Gram
            per_iter += 2 * m          # one entry of the symmetric square
    per_iter += 2 * m * m * n          # B X
    assert ref.step_flops(r, c, 5) == 5 * per_iter


# ---- tensor-parallel local update

@pytest.mark.parametrize("rows,cols,ranks", [(8, 12, 2), (7, 5, 3), (5, 16, 4), (3, 2, 3), (1, 9, 1)])
@pytest.mark.parametrize("kind", ["column", "row"])
def test_tp_shards_partition_the_weight(rows, cols, ranks, kind):
    count = np.zeros((rows, cols), dtype=int)
    sizes = []
    for rs, cs in ref.tp_shard_ranges(rows, cols, ranks, kind):
        count[rs, cs] += 1
        sizes.append((rs.stop - rs.start) if kind == "column" else (cs.stop - cs.start))
        # the split dimension is the output one (rows) for column-parallel
        # layers and the input one (cols) for row-parallel layers
        if kind == "column":
            assert (cs.start, cs.stop) == (0, cols)
        else:
            assert (rs.start, rs.stop) == (0, rows)
    assert (count == 1).all()
    assert max(sizes) - min(sizes) <= 1 and sum(sizes) == (rows if kind == "column" else cols)


@pytest.mark.parametrize("kind", ["column", "row"])
def test_shard_updates_reassemble_the_whole_matrix_sum(kind):
    rng = np.random.default_rng(7)
    W = rng.standard_normal((6, 10))
    dW = rng.standard_normal((6, 10))
    out = np.full_like(W, np.nan)
    for rs, cs in ref.tp_shard_ranges(6, 10, 4, kind):
        out[rs, cs] = ref.apply_shard(W[rs, cs].copy(), dW[rs, cs])
    for i in range(6):                       # brute force, element by element
        for j in range(10):
            assert out[i, j] == W[i, j] + dW[i, j]


def _bf16_round_once(x):
    """float64 -> the nearest bf16 value (ties to even), in one rounding."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def test_fp32_sum_then_bf16_store_is_the_exactly_rounded_sum():
    """The shard kernel adds two bf16 values in fp32 and rounds the sum once to
    bf16. That equals rounding the exact sum once: either the fp32 sum is exact
    (exponents within 16 of each other), or the smaller term is far below half
    a bf16 unit of the larger. Checked here on random pairs with every exponent
    gap up to 30, signs mixed (cancellation included), and on halfway cases."""
    from matrix_optimizer_step_muon_amd import workloads as wl
    rng = np.random.default_rng(11)
    n = 400_000
    a = _bf16_round_once(rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n)))
    gap = rng.integers(0, 31, n).astype(float)
    b = _bf16_round_once(rng.standard_normal(n) * np.abs(a) * np.exp2(-gap))
    # halfway cases: b = half a bf16 unit of a (and just above or below it)
    ulp = np.exp2(np.frexp(a)[1] - 8)
    b[:3000] = 0.5 * ulp[:3000]
    b[3000:6000] = _bf16_round_once(0.5 * ulp[3000:6000] * (1 + 2.0 ** -7))
    b[6000:9000] = _bf16_round_once(0.5 * ulp[6000:9000] * (1 - 2.0 ** -8))
    fp32_then_bf16 = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(a.astype(np.float32) + b.astype(np.float32)))
    assert np.array_equal(fp32_then_bf16.astype(np.float64), _bf16_round_once(a + b))
