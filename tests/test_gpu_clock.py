"""The engine clock probe (libmiclock.so) on the GPU: its window spans the
real time asked for, and the clock it reports is within the part's range."""

import time

import pytest
import torch

from exact_io_aware_attn_amd import clock

DEV = "cuda:0"


@pytest.mark.gpu
def test_clock_probe_idle_window():
    probe = clock.ClockProbe(n_groups=16, device=DEV)
    side = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(side):
        e0.record(side)
        probe.start(2e-3, warm_s=0.5e-3, stream=side)
        e1.record(side)
    torch.cuda.synchronize()
    o = probe.out.cpu()
    assert (o[:, 1] >= 200_000).all(), o            # window >= 2 ms of 100 MHz ticks
    assert ((o[:, 2] - o[:, 3]) >= 50_000).all(), o  # warm-up >= 0.5 ms
    mhz = probe.result()
    assert all(100.0 < m < 3000.0 for m in mhz), mhz
    # the kernel lasted at least the warm-up plus the window in event time
    assert e0.elapsed_time(e1) >= 2.4, e0.elapsed_time(e1)


@pytest.mark.gpu
def test_clock_probe_runs_beside_other_work():
    """A probe on a second stream while matrix products run on the first: it
    ends, and its window covers the real time asked for."""
    probe = clock.ClockProbe(n_groups=8, device=DEV)
    side = torch.cuda.Stream()
    x = torch.randn(4096, 4096, device=DEV)
    torch.cuda.synchronize()
    probe.start(5e-3, stream=side)
    t = time.perf_counter()
    while time.perf_counter() - t < 0.02:
        x = (x @ x) * 1e-4
    torch.cuda.synchronize()
    o = probe.out.cpu()
    assert (o[:, 1] >= 500_000).all(), o
    assert all(100.0 < m < 3000.0 for m in probe.result())
