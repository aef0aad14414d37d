"""The MFMA throughput probe (muon_mfma_probe) runs and returns finite sums.
It is a measurement aid of the bench; its rate is not checked here."""
import pytest

from matrix_optimizer_step_muon_amd import muon as mu

from gpu_helpers import log

pytestmark = pytest.mark.gpu


def test_probe_runs_and_writes_every_lane():
    import torch
    log("case mfma probe")
    blocks = 8
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    mu.mfma_probe(out, blocks, 50)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    with pytest.raises(mu.MuonError):
        mu.mfma_probe(out, blocks + 1, 50)       # out too small for the grid
