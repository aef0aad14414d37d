"""ctypes binding of libmuon.so (include/muon.h), with the same names.

It only marshals arguments: every step of the optimizer runs in the HIP
library. PyTorch supplies device memory and the current stream. If the library
is missing, the binding raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Iterable, List, Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "_lib", "libmuon.so")

MUON_OK = 0
STATUS_NAMES = {0: "OK", -1: "INVALID_ARG", -2: "ALIAS", -3: "ALIGN", -4: "UNSUPPORTED",
                -5: "HIP", -6: "OOM"}
MUON_F32, MUON_BF16, MUON_BF16_F32_MASTER = 0, 1, 2
KERNEL_KINDS = ("momentum", "norm", "gram", "square", "update", "apply", "gram_reduce")
MUON_K_COUNT = len(KERNEL_KINDS)


class muon_matrix(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("g", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("delta", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class muon_shard(ctypes.Structure):
    _fields_ = [("p", ctypes.c_void_p), ("d", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ldp", ctypes.c_int64), ("ldd", ctypes.c_int64)]


class muon_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta", ctypes.c_float), ("eps", ctypes.c_float),
                ("a", ctypes.c_float), ("b", ctypes.c_float), ("c", ctypes.c_float),
                ("ns_steps", ctypes.c_int32), ("nesterov", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class MuonError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"muon: {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None

# Every function the header declares.
EXPORTS = ("muon_hparams_default", "muon_plan", "muon_plan_workspace_bytes", "muon_step",
           "muon_plan_destroy", "muon_last_error", "muon_plan_set_timing",
           "muon_plan_kernel_times", "muon_plan_reset_timing", "muon_plan_info",
           "muon_apply_plan", "muon_apply", "muon_apply_plan_destroy",
           "muon_dp_partition_static", "muon_dp_partition", "muon_tp_micro_groups", "muon_mfma_probe",
           "muon_step_noalloc")


def lib() -> ctypes.CDLL:
    """The loaded library. It raises if libmuon.so has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m matrix_optimizer_step_muon_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    c_int, c_i32, c_i64, c_vp = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    L.muon_hparams_default.argtypes = [ctypes.POINTER(muon_hparams)]
    L.muon_plan.argtypes = [ctypes.POINTER(muon_matrix), c_i32, ctypes.POINTER(muon_hparams),
                            ctypes.POINTER(c_vp)]
    L.muon_plan_workspace_bytes.argtypes = [c_vp, ctypes.POINTER(ctypes.c_size_t)]
    L.muon_step.argtypes = [c_vp, c_vp]
    L.muon_plan_destroy.argtypes = [c_vp]
    L.muon_last_error.argtypes = []
    L.muon_last_error.restype = ctypes.c_char_p
    L.muon_plan_set_timing.argtypes = [c_vp, c_i32]
    L.muon_plan_kernel_times.argtypes = [c_vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_i64)]
    L.muon_plan_reset_timing.argtypes = [c_vp]
    L.muon_plan_info.argtypes = [c_vp, ctypes.POINTER(c_i64), ctypes.POINTER(c_i64)]
    L.muon_apply_plan.argtypes = [ctypes.POINTER(muon_shard), c_i32, c_i32, ctypes.POINTER(c_vp)]
    L.muon_apply.argtypes = [c_vp, c_vp]
    L.muon_apply_plan_destroy.argtypes = [c_vp]
    part = [ctypes.POINTER(c_i64), ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_i32), c_i32, c_i32]
    L.muon_dp_partition_static.argtypes = part + [ctypes.POINTER(c_i32), ctypes.POINTER(ctypes.c_double)]
    L.muon_dp_partition.argtypes = part + [ctypes.c_double, ctypes.POINTER(c_i32), ctypes.POINTER(ctypes.c_double)]
    L.muon_mfma_probe.argtypes = [c_vp, c_i32, c_i32, c_vp]
    L.muon_step_noalloc.argtypes = [ctypes.POINTER(muon_matrix), c_i32, ctypes.POINTER(muon_hparams), c_vp]
    L.muon_tp_micro_groups.argtypes = [ctypes.POINTER(ctypes.c_double), c_i32, c_i32, ctypes.c_double,
                                       ctypes.POINTER(c_i32), ctypes.POINTER(c_i32), ctypes.POINTER(c_i32),
                                       ctypes.POINTER(c_i32)]
    for name in EXPORTS:
        if name != "muon_last_error":
            getattr(L, name).restype = c_int
    _lib = L
    return L


def last_error() -> str:
    return lib().muon_last_error().decode()


def check(status: int) -> None:
    if status != MUON_OK:
        raise MuonError(status, last_error())


def hparams_default() -> muon_hparams:
    hp = muon_hparams()
    check(lib().muon_hparams_default(ctypes.byref(hp)))
    return hp


def make_hparams(lr=0.02, beta=0.95, eps=1e-7, coeffs=(3.4445, -4.7750, 2.0315),
                 ns_steps=5, nesterov=True, dtype=MUON_BF16) -> muon_hparams:
    a, b, c = coeffs
    return muon_hparams(lr, beta, eps, a, b, c, int(ns_steps), int(bool(nesterov)), int(dtype))


def plan_raw(descs: Sequence[muon_matrix], hp: muon_hparams) -> int:
    """muon_plan over raw descriptors; returns the plan handle (an int)."""
    arr = (muon_matrix * max(len(descs), 1))(*descs)
    out = ctypes.c_void_p()
    check(lib().muon_plan(arr, len(descs), ctypes.byref(hp), ctypes.byref(out)))
    return out.value


def step_raw(handle: int, stream: int = 0) -> None:
    check(lib().muon_step(ctypes.c_void_p(handle), ctypes.c_void_p(stream)))


def destroy_raw(handle: Optional[int]) -> None:
    check(lib().muon_plan_destroy(ctypes.c_void_p(handle)))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MUON_BF16
    if t.dtype == torch.float32:
        return MUON_F32
    raise MuonError(-4, f"unsupported tensor dtype {t.dtype}")


def _batch_dtype(W, G, M, D) -> int:
    """The plan dtype of one matrix's tensors: all bf16, all fp32, or fp32 W,
    M and delta with a bf16 G (fp32 master weights)."""
    import torch
    codes = {_dtype_code(t) for t in (W, M, D) if t is not None}
    g = _dtype_code(G)
    if codes == {g}:
        return g
    if codes == {MUON_F32} and g == MUON_BF16:
        return MUON_BF16_F32_MASTER
    raise MuonError(-1, "W, M and delta must share G's dtype, or be fp32 with a bf16 G")


def plan(mats: Iterable[Sequence], *, dtype: Optional[int] = None, **hparams) -> "Plan":
    """``Plan(mats, **hparams)``, checking that the tensors' dtypes give
    ``dtype`` (MUON_F32, MUON_BF16 or MUON_BF16_F32_MASTER) when it is given."""
    p = Plan(mats, **hparams)
    if dtype is not None and p.hparams.dtype != dtype:
        got = p.hparams.dtype
        p.close()
        raise MuonError(-1, f"the tensors give dtype {got}, not {dtype}")
    return p


def _descriptors(mats: Iterable[Sequence]):
    """Descriptors of a batch of ``(W, G, M[, delta])`` device tensors, the
    batch's dtype code and the tensors themselves."""
    tensors: List = []
    descs = []
    dtype = None
    for entry in mats:
        W, G, M = entry[0], entry[1], entry[2]
        D = entry[3] if len(entry) > 3 else None
        ref = W if W is not None else D
        for t in (W, G, M, D):
            if t is None:
                continue
            if not t.is_cuda or not t.is_contiguous() or t.dim() != 2:
                raise MuonError(-1, "tensors must be contiguous 2-D device tensors")
            if tuple(t.shape) != tuple(ref.shape):
                raise MuonError(-1, "the tensors of a matrix must share one shape")
        code = _batch_dtype(W, G, M, D)
        if dtype is not None and code != dtype:
            raise MuonError(-1, "every matrix of a batch must have the same dtypes")
        dtype = code
        tensors.append((W, G, M, D))
        descs.append(muon_matrix(W.data_ptr() if W is not None else None, G.data_ptr(),
                                 M.data_ptr(), D.data_ptr() if D is not None else None,
                                 ref.shape[0], ref.shape[1]))
    if not descs:
        raise MuonError(-1, "empty batch")
    return descs, dtype, tensors


def step_noalloc(mats: Iterable[Sequence], stream=None, *, lr=0.02, beta=0.95, eps=1e-7,
                 coeffs=(3.4445, -4.7750, 2.0315), ns_steps=5, nesterov=True) -> None:
    """muon_step_noalloc over a batch of ``(W, G, M[, delta])`` device tensors
    (as for Plan): one step in the library's static scratch, with no plan and
    no allocation, enqueued on ``stream`` (default: the current stream)."""
    import torch
    descs, dtype, _ = _descriptors(mats)
    hp = make_hparams(lr, beta, eps, coeffs, ns_steps, nesterov, dtype)
    if stream is None:
        stream = torch.cuda.current_stream()
    arr = (muon_matrix * len(descs))(*descs)
    check(lib().muon_step_noalloc(arr, len(descs), ctypes.byref(hp),
                                  ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))))


class Plan:
    """A static plan over a batch of ``(W, G, M[, delta])`` device tensors.

    Tensors must be 2-D, contiguous and on one GPU: all bf16, all fp32, or fp32
    W, M and delta with a bf16 G (fp32 master weights), the same for every
    matrix. They stay referenced by the plan, since it keeps their addresses.
    """

    def __init__(self, mats: Iterable[Sequence], *, lr=0.02, beta=0.95, eps=1e-7,
                 coeffs=(3.4445, -4.7750, 2.0315), ns_steps=5, nesterov=True):
        self._handle = None
        descs, dtype, self._tensors = _descriptors(mats)
        self.hparams = make_hparams(lr, beta, eps, coeffs, ns_steps, nesterov, dtype)
        self._handle = plan_raw(descs, self.hparams)

    def step(self, stream=None) -> None:
        import torch
        if stream is None:
            stream = torch.cuda.current_stream()
        step_raw(self._handle, stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))

    def workspace_bytes(self) -> int:
        v = ctypes.c_size_t()
        check(lib().muon_plan_workspace_bytes(ctypes.c_void_p(self._handle), ctypes.byref(v)))
        return v.value

    def info(self):
        t = (ctypes.c_int64 * MUON_K_COUNT)()
        g = (ctypes.c_int64 * MUON_K_COUNT)()
        check(lib().muon_plan_info(ctypes.c_void_p(self._handle), t, g))
        return {k: {"tiles": t[i], "grid": g[i]} for i, k in enumerate(KERNEL_KINDS)}

    def set_timing(self, enable: bool) -> None:
        check(lib().muon_plan_set_timing(ctypes.c_void_p(self._handle), int(bool(enable))))

    def kernel_times(self):
        """Per kernel kind: (total ms, launches), from HIP events on the step stream."""
        ms = (ctypes.c_double * MUON_K_COUNT)()
        n = (ctypes.c_int64 * MUON_K_COUNT)()
        check(lib().muon_plan_kernel_times(ctypes.c_void_p(self._handle), ms, n))
        return {k: (ms[i], n[i]) for i, k in enumerate(KERNEL_KINDS)}

    def reset_timing(self) -> None:
        check(lib().muon_plan_reset_timing(ctypes.c_void_p(self._handle)))

    def close(self) -> None:
        if self._handle is not None:
            h, self._handle = self._handle, None
            destroy_raw(h)
        self._tensors = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


class ApplyPlan:
    """A static plan of the tensor-parallel local update P += Delta W over a
    list of ``(P, D)`` device tensors: 2-D, one dtype (bf16 or fp32), unit
    column stride (row-major views, such as a column block of a larger matrix,
    are fine). P is updated in place; D is read. The plan keeps the tensors
    referenced, since it keeps their addresses."""

    def __init__(self, pairs: Iterable[Sequence]):
        self._handle = None
        self._tensors: List = []
        descs = []
        dtype = None
        for P, D in pairs:
            for t in (P, D):
                if not t.is_cuda or t.dim() != 2 or t.stride(1) != 1:
                    raise MuonError(-1, "shards must be 2-D device tensors with unit column stride")
            code = _dtype_code(P)
            dtype = code if dtype is None else dtype
            if _dtype_code(D) != dtype or code != dtype or tuple(P.shape) != tuple(D.shape):
                raise MuonError(-1, "P and D of every shard must share one dtype and shape")
            self._tensors.append((P, D))
            descs.append(muon_shard(P.data_ptr(), D.data_ptr(), P.shape[0], P.shape[1],
                                    P.stride(0), D.stride(0)))
        if not descs:
            raise MuonError(-1, "no shards")
        arr = (muon_shard * len(descs))(*descs)
        out = ctypes.c_void_p()
        check(lib().muon_apply_plan(arr, len(descs), dtype, ctypes.byref(out)))
        self._handle = out.value

    def apply(self, stream=None) -> None:
        import torch
        if stream is None:
            stream = torch.cuda.current_stream()
        check(lib().muon_apply(ctypes.c_void_p(self._handle),
                               ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))))

    def close(self) -> None:
        if self._handle is not None:
            h, self._handle = self._handle, None
            check(lib().muon_apply_plan_destroy(ctypes.c_void_p(h)))
        self._tensors = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def dp_partition(buckets: Sequence[Sequence[int]], ranks: int, alpha: Optional[float] = 1.0,
                 loads: Optional[Sequence[Sequence[float]]] = None):
    """Data-parallel static partition of a parameter buffer (host only).

    ``buckets``: per bucket, the element counts of its parameters in buffer
    order. ``loads``: the same shape, each parameter's load (default: its
    element count). ``alpha``: the alpha-Balanced Greedy LPT algorithm with that
    alpha, or None for the Start_Index rule without load balancing. Returns
    ``(cuts, rank_loads)``: per bucket the ranks + 1 parameter-index cuts (rank
    r owns parameters cuts[r] .. cuts[r+1] - 1), and each rank's total load."""
    lens = [len(b) for b in buckets]
    flat = [int(x) for b in buckets for x in b]
    n, nb = len(flat), len(lens)
    sz = (ctypes.c_int64 * max(n, 1))(*flat)
    ld = None
    if loads is not None:
        fl = [float(x) for b in loads for x in b]
        if len(fl) != n:
            raise MuonError(-1, "loads must have the shape of buckets")
        ld = (ctypes.c_double * max(n, 1))(*fl)
    bl = (ctypes.c_int32 * max(nb, 1))(*lens)
    cuts = (ctypes.c_int32 * max(nb * (ranks + 1), 1))()
    rl = (ctypes.c_double * max(ranks, 1))()
    if alpha is None:
        check(lib().muon_dp_partition_static(sz, ld, bl, nb, ranks, cuts, rl))
    else:
        check(lib().muon_dp_partition(sz, ld, bl, nb, ranks, float(alpha), cuts, rl))
    out = [list(cuts[i * (ranks + 1):(i + 1) * (ranks + 1)]) for i in range(nb)]
    return out, list(rl[:ranks])


def tp_micro_groups(costs: Sequence[float], ranks: int, c_max: float):
    """TP micro-group schedule (host only). Returns the groups in order, each
    as ``(tensor IDs, host ranks)``, the IDs in schedule order."""
    n = len(costs)
    c = (ctypes.c_double * max(n, 1))(*[float(x) for x in costs])
    order = (ctypes.c_int32 * max(n, 1))()
    group_of = (ctypes.c_int32 * max(n, 1))()
    host_of = (ctypes.c_int32 * max(n, 1))()
    ng = ctypes.c_int32()
    check(lib().muon_tp_micro_groups(c, n, ranks, float(c_max), order, group_of, host_of, ctypes.byref(ng)))
    groups = [([], []) for _ in range(ng.value)]
    for i in order[:n]:
        groups[group_of[i]][0].append(i)
        groups[group_of[i]][1].append(host_of[i])
    return groups


def mfma_probe(out, blocks: int, iters: int, stream=None) -> None:
    """Enqueues the MFMA throughput probe: ``blocks`` workgroups, each wave
    issuing ``iters`` * 8 bf16 32x32x16 MFMAs; ``out`` is a float32 device
    tensor of at least blocks * 256 elements."""
    import torch
    if out.dtype != torch.float32 or not out.is_cuda or out.numel() < blocks * 256:
        raise MuonError(-1, "out must be a float32 device tensor of blocks * 256 elements")
    if stream is None:
        stream = torch.cuda.current_stream()
    check(lib().muon_mfma_probe(ctypes.c_void_p(out.data_ptr()), int(blocks), int(iters),
                                ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))))
