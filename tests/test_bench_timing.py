"""The benchmark's timing helpers: the clock sampler's summary (host only) and the fence-free
per-kernel events against the step time (GPU)."""
import pytest

import bench


def _sampler(samples):
    c = bench.ClockSampler.__new__(bench.ClockSampler)  # no amdsmi handle: only the summary is used
    c.samples = samples
    return c


def test_clock_summary_skips_the_first_readings():
    """Readings taken before SKIP_S (the firmware's figure can trail a change of load) are left
    out; the median, range and count are those of the later readings."""
    skip = bench.ClockSampler.SKIP_S
    s = _sampler([(0.0, 170.0), (skip / 2, 170.0), (skip, 2100.0), (skip + 0.01, 2400.0), (skip + 0.02, 2300.0)])
    out = s.summary()
    assert out["samples"] == 3 and out["min_mhz"] == 2100.0 and out["max_mhz"] == 2400.0
    assert out["median_mhz"] == 2300.0
    assert out["window_s"] == round(skip + 0.02, 3)


def test_clock_summary_without_late_readings_is_none():
    assert _sampler([(0.0, 2400.0), (0.01, 2400.0)]).summary() is None
    assert _sampler([]).summary() is None


@pytest.mark.gpu
def test_kernel_events_time_each_kernel_of_the_step():
    """TimedSteps with fence-free events on every step of a small causal fwd+bwd: every kernel's
    average is positive and the three add up to about the step time (the events sit between the
    kernels, so their sum can exceed the step time only by the few dispatch gaps they split)."""
    import torch

    from io_aware_flashattention_flash_amd import inputs

    dev = torch.device("cuda:0")
    w = inputs.Workload("small", "bf16", 2, 8, 512, 64, True, True, 1.0)
    step = bench.prepare_fwdbwd(w, inputs.make_inputs(w), dev, lambda a, dt: torch.from_numpy(a).to(dev).to(dt))
    for _ in range(20):
        step()
    timed = bench.TimedSteps(step, 50, sample_every=1)
    assert all(isinstance(e, bench.KernelEvent) for evs in timed.kev.values() for e in evs)
    timed.enqueue()
    ms_step, kern = timed.result()
    assert set(kern) == {"fwd", "bwd_dq", "bwd_dkdv"}
    assert all(v > 0 for v in kern.values()), kern
    total = sum(kern.values())
    assert 0.5 * ms_step < total < ms_step + 0.03, (ms_step, kern)
