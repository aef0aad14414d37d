import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side oracle run")


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped only when no GPU is visible at all. With a GPU, a
    # missing or broken library makes them fail, never fall back.
    if any("gpu" in item.keywords for item in items) and not _gpu_visible():
        skip = pytest.mark.skip(reason="no GPU visible")
        for item in items:
            if "gpu" in item.keywords:
                item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """After a GPU run, the relative Frobenius errors against the oracle: every
    full-size matrix, and the worst matrix of every other case."""
    helpers = sys.modules.get("gpu_helpers")
    records = getattr(helpers, "RECORDS", None)
    if not records:
        return
    tr = terminalreporter
    tr.write_line("")
    tr.write_line("parity against the fp64 oracle (relFro; bars: bf16 2e-2, fp32 1e-4)")
    fmt = lambda errs: " ".join(f"{k}={v:.2e}" for k, v in errs.items())
    worst = {}
    for label, shape, errs, tol, full in records:
        if full:
            continue
        w = worst.setdefault(label, [shape, {}, tol])
        if max(errs.values(), default=0.0) >= max(w[1].values(), default=-1.0):
            w[0], w[1] = shape, errs
    for label, (shape, errs, tol) in worst.items():
        tr.write_line(f"  {label}: worst {shape[0]}x{shape[1]} {fmt(errs)} (bar {tol:g})")
    for label, shape, errs, tol, full in records:
        if full:
            tr.write_line(f"  {label} {shape[0]}x{shape[1]}: {fmt(errs)} (bar {tol:g})")
