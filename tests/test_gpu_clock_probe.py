"""The engine-clock probe that the benchmark reports (birkhoff_clock_probe):
its counts are filled, and the clock it yields lies between the chip's idle and
peak engine clocks.  A measurement aid, not part of the projection."""
import pytest

torch = pytest.importorskip("torch")
import birkhoff_projection_amd as bp  # noqa: E402

pytestmark = pytest.mark.gpu


def test_clock_probe_reads_a_plausible_clock():
    dev = torch.device("cuda:0")
    probe = bp.ClockProbe(dev, blocks=64, ticks=2000)
    probe.launch()
    torch.cuda.synchronize()
    c = probe.counts.view(-1, 2).cpu()
    assert (c[:, 1] >= 2000).all(), c[:, 1].min()      # every workgroup ran its full interval
    assert (c[:, 0] > 0).all()
    assert probe.wall_khz > 0
    mhz = probe.mhz()
    print("clock probe: %.0f MHz (constant counter %d kHz)" % (mhz, probe.wall_khz))
    assert 50.0 <= mhz <= 2500.0, mhz


def test_clock_probe_on_a_side_stream():
    dev = torch.device("cuda:0")
    s = torch.cuda.Stream(device=dev)
    probe = bp.ClockProbe(dev, blocks=8, ticks=500)
    probe.launch(s)
    s.synchronize()
    assert 50.0 <= probe.mhz() <= 2500.0
