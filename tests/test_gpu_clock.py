"""The measurement clock sampler: workgroups spread over the compute units, each writing its own
unit's counters, so that a unit's two samples give its clock."""
import statistics

import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def test_clock_sample_pairs_per_compute_unit():
    import bench
    a = torch.randn(4096, 4096, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        torch.mul(a, 1.0001, out=b)   # warm-up: allocations and first launches before the samples
    torch.cuda.synchronize()
    clk = bench.DeviceClock(torch.cuda.current_stream().cuda_stream)
    clk.start()
    for _ in range(200):
        torch.mul(a, 1.0001, out=b)   # back-to-back work between the samples (a few ms)
    clk.stop()
    torch.cuda.synchronize()
    units = clk.per_unit()
    mhz = sorted(m for m, _ in units)
    print(f"{len(units)} units; clock min {mhz[0]:.0f}, median {statistics.median(mhz):.0f}, "
          f"max {mhz[-1]:.0f} MHz; summary {clk.summary()}", flush=True)
    assert len(units) >= 200                      # most of the 256 compute units are reached
    # a busy interval runs near the shader clock (at most 2.4 GHz on this part), on every unit
    assert all(300.0 < m < 2600.0 for m in mhz), (mhz[:5], mhz[-5:])
