"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, and run the fp64 oracle on the same stored bits."""

from __future__ import annotations

import sys
import time

import numpy as np

from matrix_optimizer_step_muon_amd import muon as mu
from matrix_optimizer_step_muon_amd import workloads as wl
from oracle import muon_ref as ref

TOL = {"bf16": 2e-2, "f32": 1e-4}

# Every comparison made in this session: (label, shape, {"O": .., "M": .., "W": ..},
# tolerance, full_size). tests/conftest.py prints them at the end of the run.
RECORDS = []


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_device(a: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_host(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def gpu_step(inputs, dtype: str, hp: dict, *, with_delta=True, with_w=True, steps=1, order=None,
             grads=None):
    """Runs `steps` steps of the HIP path. Returns per matrix (W', M', delta)
    as storage arrays. `grads[s]` replaces the gradients for step s > 0."""
    import torch
    order = list(range(len(inputs))) if order is None else list(order)
    dev = []
    for (W, G, M) in inputs:
        Wd = to_device(W, dtype) if with_w else None
        Dd = torch.empty_like(to_device(G, dtype)) if with_delta else None
        if Dd is not None:
            Dd.fill_(float("nan"))   # any element the step fails to write shows up
        dev.append([Wd, to_device(G, dtype), to_device(M, dtype), Dd])
    plan = mu.Plan([dev[i] for i in order], **hp)
    for s in range(steps):
        if s > 0 and grads is not None:
            for i, G in enumerate(grads[s]):
                dev[i][1].copy_(to_device(G, dtype))
        plan.step()
    torch.cuda.synchronize()
    out = [(to_host(d[0], dtype) if d[0] is not None else None, to_host(d[2], dtype),
            to_host(d[3], dtype) if d[3] is not None else None) for d in dev]
    plan.close()
    return out


def oracle_step(inputs, dtype: str, hp: dict, steps=1, grads=None):
    """fp64 oracle on the exact stored values. Returns (W', M', O) per matrix."""
    res = []
    for i, (W, G, M) in enumerate(inputs):
        Wf, Gf, Mf = (wl.stored_to_f64(x, dtype) for x in (W, G, M))
        O = None
        for s in range(steps):
            if s > 0 and grads is not None:
                Gf = wl.stored_to_f64(grads[s][i], dtype)
            Wf, Mf, O = ref.muon_step(Wf, Gf, Mf, **hp)
        res.append((Wf, Mf, O))
    return res


def compare(gpu, want, dtype: str, hp: dict, inputs, label: str, tol=None, full_size=False):
    """relFro of O (from delta), M' and W' against the oracle, per matrix.
    Returns the worst of each and asserts them against the tolerance. Every
    result is also recorded in RECORDS (full_size marks the full-size cases,
    which the end-of-run summary lists matrix by matrix)."""
    tol = TOL[dtype] if tol is None else tol
    worst = {"O": 0.0, "M": 0.0, "W": 0.0}
    for i, ((Wg, Mg, Dg), (Wr, Mr, Or)) in enumerate(zip(gpu, want)):
        r, c = inputs[i][0].shape
        ls = hp["lr"] * ref.update_scale(r, c)
        errs = {"M": wl.rel_fro(wl.stored_to_f64(Mg, dtype), Mr)}
        if Dg is not None:
            D = wl.stored_to_f64(Dg, dtype)
            assert np.isfinite(D).all(), f"{label} matrix {i}: non-finite delta"
            errs["O"] = wl.rel_fro(-D / ls, Or) if ls != 0 else 0.0
        if Wg is not None:
            errs["W"] = wl.rel_fro(wl.stored_to_f64(Wg, dtype), Wr)
        for k, v in errs.items():
            worst[k] = max(worst[k], v)
        RECORDS.append((label, (r, c), dict(errs), tol, full_size))
        log(f"{label} matrix {i} {r}x{c}: " + " ".join(f"relFro({k})={v:.3e}" for k, v in errs.items()))
        for k, v in errs.items():
            assert v <= tol, f"{label} matrix {i} ({r}x{c}): relFro({k}) = {v:.3e} > {tol}"
    return worst
