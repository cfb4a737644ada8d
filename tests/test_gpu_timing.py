"""The benchmark's timing-only events (HIP events created with
hipEventDisableSystemFence, bench.TimingEvent) against torch's default
events around the same spinning kernel: both pairs see its length."""
import pytest
import torch

from gpu_harness import say

pytestmark = pytest.mark.gpu


def test_timing_event_measures_a_spinning_kernel():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    say("timing-only events around a spinning kernel")
    stream = torch.cuda.current_stream()
    cycles = 480_000  # a few hundred microseconds at the shader clock
    torch.cuda._sleep(1000)
    torch.cuda.synchronize()
    ours = [bench.TimingEvent() for _ in range(2)]
    theirs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ours[0].record(stream)
    torch.cuda._sleep(cycles)
    ours[1].record(stream)
    theirs[0].record(stream)
    torch.cuda._sleep(cycles)
    theirs[1].record(stream)
    torch.cuda.synchronize()
    t_ours = ours[0].elapsed_time(ours[1]) * 1e3
    t_theirs = theirs[0].elapsed_time(theirs[1]) * 1e3
    assert t_ours > 50.0 and t_theirs > 50.0, (t_ours, t_theirs)
    assert abs(t_ours - t_theirs) < 0.2 * t_theirs, (t_ours, t_theirs)
