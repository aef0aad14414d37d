"""Seeded synthetic inputs for the whole-tensor Muon step.

Both sides of every parity check use this module: the HIP path and the fp64
oracle. It holds none of the method's arithmetic: it only draws random
matrices, converts them to their storage format (fp32, or bf16 by
round-to-nearest-even) and widens stored values exactly to float64.

Workloads. The Canzona pages measure Muon on the Qwen3 family, 1.7B to 32B,
with sequence length 4096 and batch 1 per DP rank (Canzona analysis page,
section 5, "Dataset"). No dataset or trained weights are involved, so every
input here is a seeded Gaussian draw at the Qwen3 projection shapes,
(out, in) row-major:
- gradients ~ N(0, 1e-3^2);
- weights ~ N(0, 0.02^2);
- momentum = one prior gradient draw, i.e. the plain-momentum state one step
  after starting from zero.

Generator: numpy PCG64 seeded with ``[workload_seed, matrix_index, kind]``
(kind 0 = G, 1 = W, 2 = the prior gradient). It draws float32 standard
normals, scales them in float32, then rounds to bf16 with round-to-nearest-even
where the storage is bf16.
"""

from __future__ import annotations

import dataclasses
from typing import List, Sequence, Tuple

import numpy as np

KIND_G, KIND_W, KIND_GPREV = 0, 1, 2

# Qwen3-1.7B decoder-layer projections: q, k, v, o, gate, up, down (rows x cols).
QWEN3_1P7B_LAYER = [(2048, 2048), (1024, 2048), (1024, 2048), (2048, 2048),
                    (6144, 2048), (6144, 2048), (2048, 6144)]
# Qwen3-32B decoder-layer projections, unsharded.
QWEN3_32B_LAYER = [(8192, 5120), (1024, 5120), (1024, 5120), (5120, 8192),
                   (25600, 5120), (25600, 5120), (5120, 25600)]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dtype: str                       # "f32" or "bf16" storage of W, G, M
    shapes: Tuple[Tuple[int, int], ...]
    g_std: float
    w_std: float
    momentum: str                    # "zero" or "prev" (one prior gradient draw)
    lr: float = 0.02
    beta: float = 0.95
    nesterov: bool = True
    ns_steps: int = 5

    @property
    def numel(self) -> int:
        return sum(r * c for r, c in self.shapes)

    def hparams(self) -> dict:
        return dict(lr=self.lr, beta=self.beta, nesterov=self.nesterov,
                    ns_steps=self.ns_steps)


WORKLOADS = {
    "tiny_f32_16x128x256": Workload(
        "tiny_f32_16x128x256", 1, "f32", tuple([(128, 256)] * 16),
        g_std=1.0, w_std=1.0, momentum="zero"),
    "qwen3_1p7b_layer": Workload(
        "qwen3_1p7b_layer", 2, "bf16", tuple(QWEN3_1P7B_LAYER),
        g_std=1e-3, w_std=0.02, momentum="prev"),
    "qwen3_1p7b_28_layers": Workload(
        "qwen3_1p7b_28_layers", 3, "bf16", tuple(QWEN3_1P7B_LAYER * 28),
        g_std=1e-3, w_std=0.02, momentum="prev"),
    "qwen3_32b_layer": Workload(
        "qwen3_32b_layer", 4, "bf16", tuple(QWEN3_32B_LAYER),
        g_std=1e-3, w_std=0.02, momentum="prev"),
    "qwen3_32b_rank_share": Workload(
        "qwen3_32b_rank_share", 5, "bf16",
        tuple(QWEN3_32B_LAYER * 2 + [(1024, 5120), (1024, 5120), (25600, 5120)]),
        g_std=1e-3, w_std=0.02, momentum="prev"),
}


def custom_workload(name: str, shapes: Sequence[Tuple[int, int]], dtype: str,
                    seed: int = 1000, g_std: float = 1e-3, w_std: float = 0.02,
                    momentum: str = "prev", **hp) -> Workload:
    return Workload(name, seed, dtype, tuple(tuple(s) for s in shapes),
                    g_std=g_std, w_std=w_std, momentum=momentum, **hp)


# ---------------------------------------------------------------- bf16 storage

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even; NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored array (float32, or uint16 bf16 bits)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float array -> storage array (float32, or uint16 bf16 bits)."""
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f32":
        return np.ascontiguousarray(x32)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# ----------------------------------------------------------------- generators

def draw(seed: int, index: int, kind: int, shape: Tuple[int, int], std: float) -> np.ndarray:
    """One seeded N(0, std^2) float32 matrix."""
    rng = np.random.default_rng([seed, index, kind])
    x = rng.standard_normal(shape, dtype=np.float32)
    x *= np.float32(std)
    return x


def generate_matrix(wl: Workload, index: int):
    """Storage arrays ``(W, G, M)`` of matrix ``index`` of a workload."""
    shape = wl.shapes[index]
    G = to_storage(draw(wl.seed, index, KIND_G, shape, wl.g_std), wl.dtype)
    W = to_storage(draw(wl.seed, index, KIND_W, shape, wl.w_std), wl.dtype)
    if wl.momentum == "zero":
        M = to_storage(np.zeros(shape, np.float32), wl.dtype)
    elif wl.momentum == "prev":
        M = to_storage(draw(wl.seed, index, KIND_GPREV, shape, wl.g_std), wl.dtype)
    else:
        raise ValueError(f"unknown momentum init {wl.momentum!r}")
    return W, G, M


def generate(wl: Workload, indices: Sequence[int] | None = None) -> List[tuple]:
    """Storage arrays ``(W, G, M)`` for the chosen matrices (all by default)."""
    if indices is None:
        indices = range(len(wl.shapes))
    return [generate_matrix(wl, i) for i in indices]


def rel_fro(x: np.ndarray, ref: np.ndarray) -> float:
    """``||x - ref||_F / ||ref||_F`` in float64 (0 when both are zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    if den == 0.0:
        return float(num)
    return float(num / den)


# ------------------------------------------------------- parameter buffers

QWEN3_32B_HIDDEN = 5120
QWEN3_VOCAB = 151936


def qwen3_32b_param_buffer(tp: int = 1, bucket_elems: int = 40_000_000) -> List[List[Tuple[int, ...]]]:
    """Shapes of a Qwen3-32B-shaped parameter buffer, split into buckets.

    Per decoder layer: q 8192 x 5120, k and v 1024 x 5120, o 5120 x 8192, gate
    and up 25600 x 5120, down 5120 x 25600 (the shapes of the Qwen3-32B layer
    workload), the q and k norms (128) and the two layer norms (5120); 64
    layers, the input embedding and the output projection (vocabulary x 5120)
    and the final norm. With tp > 1 this is one tensor-parallel rank's local
    buffer: column-parallel weights (q, k, v, gate, up, the embeddings) keep
    1/tp of their rows, row-parallel ones (o, down) 1/tp of their columns, and
    norms are whole. Parameters enter the buffer in reverse order (the order in
    which gradients become ready) and a bucket closes once it holds at least
    bucket_elems elements; a parameter is never split."""
    H, V = QWEN3_32B_HIDDEN, QWEN3_VOCAB
    col = lambda r, c: (r // tp, c)
    row = lambda r, c: (r, c // tp)
    layer = [col(8192, H), col(1024, H), col(1024, H), row(H, 8192), col(25600, H), col(25600, H),
             row(H, 25600), (128,), (128,), (H,), (H,)]
    params = [col(V, H)] + layer * 64 + [(H,), col(V, H)]
    buckets: List[List[Tuple[int, ...]]] = [[]]
    filled = 0
    for shape in reversed(params):
        buckets[-1].append(shape)
        filled += int(np.prod(shape))
        if filled >= bucket_elems:
            buckets.append([])
            filled = 0
    if not buckets[-1]:
        buckets.pop()
    return buckets
