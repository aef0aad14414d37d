"""Plain fp64 CPU oracle of the whole-tensor Muon optimizer step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(the HIP library and its Python binding) never imports it, and this module
imports nothing from the product path.

What it computes, and where each step comes from:

* The Canzona analysis page (paper-graph-ui), section "2. Context and
  Motivation", gives the matrix-optimizer update form
  ``W_{t+1} = W_t - eta * MatrixOp(W_t, grad W_t)`` and says Muon's MatrixOp
  orthogonalises with Newton-Schulz iterations.
* The same page, section "3.4 Detailed, Sentence-Based Technical Breakdown"
  (the Atomicity Constraint), says that the orthogonalised matrix comes from
  repeated matrix products that mix every row and column of the whole gradient.
  So the step runs on the complete tensor.
* The same section ("Task abstraction" and the micro-group lifecycle, steps 2
  and 4) makes the Muon momentum buffer per-tensor optimizer state. It writes
  the step as ``Delta W = Muon_step(G, States_local)`` followed by
  ``P <- P + Delta W``.
* The pages print no Muon constants. The momentum form (plain accumulation with
  Nesterov look-ahead), the quintic Newton-Schulz coefficients
  (a, b, c) = (3.4445, -4.7750, 2.0315), the step count 5, the transpose to
  rows <= cols and the scale sqrt(max(1, rows/cols)) are the standard Muon
  method's. They are taken as given, and each reading is listed with the design
  notes.

Everything is float64 with no intermediate rounding. Inputs are the exact stored
values (fp32 or bf16) widened to float64 by the caller. numpy's float64 matmul
(a BLAS dgemm) is the one library primitive used. There is no blocking, fusion or
reordering beyond the definition.

Pins (tests/test_oracle_pins.py, all on the CPU):
- the scalar momentum example;
- a brute-force Frobenius norm and a brute-force matmul;
- the SVD closed form of the odd-polynomial iteration;
- the quintic's attracting band;
- cubic Newton-Schulz converging to the polar factor;
- transpose equivariance and scale invariance;
- semi-orthogonal and rank-1 closed forms;
- the T = 0 and zero-input special cases, and where eps sits;
- the TP partition covers every element of a weight exactly once, and the
  shard-by-shard local update reassembles the whole-matrix sum (brute force).
Every function here has at least one pin.
"""

from __future__ import annotations

import math

import numpy as np

# Quintic Newton-Schulz coefficients (a, b, c) of the standard Muon method.
# p(x) = a*x + b*x**3 + c*x**5 is applied to every singular value.
QUINTIC_COEFFS = (3.4445, -4.7750, 2.0315)
DEFAULT_NS_STEPS = 5
DEFAULT_EPS = 1e-7


def momentum_update(G: np.ndarray, M: np.ndarray, beta: float, nesterov: bool):
    """Momentum buffer update and the direction the orthogonaliser sees.

    The buffer is the Muon momentum state that stays on the rank that owns the
    tensor (Canzona analysis page, section 3.4, "Task abstraction as the
    organizing concept").

    Plain accumulation ``M' = beta*M + G``. With Nesterov the direction is
    ``U = G + beta*M'`` (the look-ahead taken from the updated buffer); without
    it, ``U = M'``. The pages leave this form open; it is the standard Muon one.
    """
    M_new = beta * M + G
    U = G + beta * M_new if nesterov else M_new
    return M_new, U


def frobenius_norm(X: np.ndarray) -> float:
    """Frobenius norm, sqrt of the sum of squares of every entry."""
    return float(np.sqrt(np.sum(X * X)))


def frobenius_normalize(X: np.ndarray, eps: float) -> np.ndarray:
    """``X / (||X||_F + eps)``.

    This bounds the largest singular value by 1, which keeps it inside the
    quintic's basin. eps only matters for an all-zero X, where it gives 0, not NaN.
    """
    return X / (frobenius_norm(X) + eps)


def newton_schulz(X: np.ndarray, steps: int, coeffs=QUINTIC_COEFFS) -> np.ndarray:
    """Fixed-count odd-polynomial Newton-Schulz iteration on a wide X (m <= n).

    Each step forms the Gram matrix ``A = X X^T`` and ``B = b*A + c*A^2``, then
    sets ``X <- a*X + B X``. On singular values this is
    ``sigma <- a*sigma + b*sigma^3 + c*sigma^5``. These are the repeated products
    that mix all rows and columns (Canzona analysis page, section 3.4, the
    Atomicity Constraint). The count is fixed and there is no convergence test.
    """
    a, b, c = coeffs
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X


def orthogonalize(U: np.ndarray, steps: int = DEFAULT_NS_STEPS,
                  coeffs=QUINTIC_COEFFS, eps: float = DEFAULT_EPS) -> np.ndarray:
    """Muon's MatrixOp: the Newton-Schulz orthogonalisation of the whole matrix U.

    A tall U (rows > cols) is transposed first, so that the Gram matrix is the
    smaller one, and transposed back at the end. In exact arithmetic the result is
    the same either way; it only changes the cost. A square U is not transposed.
    """
    tall = U.shape[0] > U.shape[1]
    X = U.T if tall else U
    X = frobenius_normalize(X, eps)
    X = newton_schulz(X, steps, coeffs)
    return X.T if tall else X


def update_scale(rows: int, cols: int) -> float:
    """Per-matrix update scale ``sqrt(max(1, rows/cols))`` for a rows x cols weight."""
    return math.sqrt(max(1.0, rows / cols))


def muon_step(W: np.ndarray, G: np.ndarray, M: np.ndarray, *, lr: float,
              beta: float, nesterov: bool = True, ns_steps: int = DEFAULT_NS_STEPS,
              coeffs=QUINTIC_COEFFS, eps: float = DEFAULT_EPS):
    """One whole-tensor Muon step on one matrix; returns ``(W', M', O)``.

    ``W' = W - lr * sqrt(max(1, rows/cols)) * O``. This is the update
    ``W_{t+1} = W_t - eta * MatrixOp`` of the Canzona analysis page (section 2),
    with ``O = orthogonalize(U)``. ``-lr * scale * O`` is the ``Delta W`` that
    the host rank produces in the micro-group lifecycle (section 3.4, step 2)
    and that step 4 adds to the parameters.
    """
    W = np.asarray(W, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    if W.ndim != 2 or W.shape != G.shape or W.shape != M.shape:
        raise ValueError("W, G and M must be matrices of one shape")
    M_new, U = momentum_update(G, M, beta, nesterov)
    O = orthogonalize(U, ns_steps, coeffs, eps)
    W_new = W - lr * update_scale(*W.shape) * O
    return W_new, M_new, O


def step_flops(rows: int, cols: int, ns_steps: int = DEFAULT_NS_STEPS) -> int:
    """Algorithmic flops of the Newton-Schulz part of one step on one matrix.

    Only the triangles the method needs are counted. With m = min(rows, cols)
    and n = max(rows, cols), one iteration is:
    - the symmetric Gram X X^T: m(m+1)/2 entries of a length-n dot product,
      so m(m+1)n flops;
    - the symmetric square A A: m^2(m+1) flops;
    - the product B X: 2 m^2 n flops.
    """
    m, n = min(rows, cols), max(rows, cols)
    return ns_steps * (m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n)


def tp_shard_ranges(rows: int, cols: int, ranks: int, kind: str):
    """The tensor-parallel partition of a rows x cols (out, in) weight over
    ``ranks`` ranks, as ``[(row_slice, col_slice)]`` per rank.

    A column-parallel layer splits the output dimension (the rows), a
    row-parallel layer the input dimension (the columns) (Canzona analysis page,
    section 2, "The Core Problem"). The pages do not say how a dimension that
    is not a multiple of the rank count is split; rank r takes
    [r*n // ranks, (r+1)*n // ranks), so sizes differ by at most one.
    """
    if kind not in ("column", "row"):
        raise ValueError("kind must be 'column' or 'row'")
    n = rows if kind == "column" else cols
    cuts = [r * n // ranks for r in range(ranks + 1)]
    out = []
    for r in range(ranks):
        part = slice(cuts[r], cuts[r + 1])
        out.append((part, slice(0, cols)) if kind == "column" else (slice(0, rows), part))
    return out


def apply_shard(P: np.ndarray, D: np.ndarray) -> np.ndarray:
    """The local update of one shard, ``P_local + Delta W_local``, element by
    element (Canzona analysis page, section 3.4, "The TP Task Abstraction",
    micro-group lifecycle step 4), in float64. The caller rounds the result to
    the storage type."""
    if P.shape != D.shape:
        raise ValueError("P and D must have one shape")
    return P + D
