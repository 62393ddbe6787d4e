"""The MFMA issue-rate probe (moe_mfma_probe) on the GPU: every wave reports its loop's cycles,
and the cycles per instruction sit at the matrix cores' issue cost (a 32x32x16 bf16 MFMA is 8
passes of 4 cycles, a 32x32x64 E4M3 MFMA-scale 16 passes), well below twice it."""
import pytest
import torch

import mixture_experts_grouped_permute_amd as m

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,cycles", [(2, 32.0), (3, 32.0), (0, 64.0), (1, 64.0), (4, 64.0)])
def test_mfma_probe_issue_cost(kind, cycles):
    r = m.mfma_probe(kind, iters=200, reps=1)
    assert r["waves"] == 1024
    assert cycles * 0.95 <= r["cycles_per_mfma_mean"] <= cycles * 1.5, r
    assert r["cycles_per_mfma_max"] <= cycles * 2.0, r
    assert 0.5 < r["clock_ghz"] < 3.0, r


def test_load_probe_patterns():
    """moe_load_probe: every pattern fills LDS at a plausible rate, and L2-resident data fills it
    faster than data streamed from HBM."""
    buf = torch.zeros(m.load().moe_load_probe_bytes(), dtype=torch.uint8, device="cuda:0")
    r = [m.load_probe(p, stages=256, reps=1, buf=buf) for p in range(4)]
    for x in r:
        assert 1.0 < x["bytes_per_cycle_per_cu"] < 256.0, x
    assert r[0]["bytes_per_cycle_per_cu"] > r[1]["bytes_per_cycle_per_cu"], r
