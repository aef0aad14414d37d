"""Whole-tensor Muon optimizer step on MI355X (gfx950).

The compute lives in the HIP library ``_lib/libmuon.so``. ``muon`` is its ctypes
binding, and ``workloads`` makes seeded synthetic inputs. The library loads on
first use, and importing the package does not touch the GPU.
"""

from .muon import (  # noqa: F401
    MUON_BF16,
    MUON_F32,
    MuonError,
    Plan,
    hparams_default,
    lib,
    make_hparams,
)

__all__ = ["Plan", "MuonError", "lib", "hparams_default", "make_hparams", "MUON_BF16", "MUON_F32"]
