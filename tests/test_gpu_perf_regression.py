"""Performance regression guard at the all-seven workload (16384 x 256).

Each estimator's per-launch time, measured as the bench measures it (rotating
buffer sets over 1 GiB, HIP events on the launch stream), must stay under a
ceiling set 1.5x above what the current kernels measure on one MI355X
(discounted returns 11.0 us, TD(lambda) / GAE 12.0 us, V-trace 18.9 us,
Retrace 20.2 us, traces / prefix sums 8.6 us), loose enough for the spread
between GPUs and runs, tight enough to catch a routing or occupancy mistake
(those have cost 1.3-2x here).
"""
from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu

CEILING_US = {
    "discounted_returns": 16.5,
    "td_lambda": 18.0,
    "gae": 18.0,
    "vtrace": 28.5,
    "retrace": 30.5,
    "eligibility_traces": 13.0,
    "episodic_prefix_sum": 13.0,
}


def test_per_estimator_time_at_16384x256():
    import torch
    import bench
    from linear_recurrence_scan_reverse_amd import synth
    w = synth.WORKLOADS["all7_16384x256"]
    d = synth.workload_inputs(w)
    runner = bench.Runner(w, d, 5, torch.device("cuda", 0))
    per = bench.time_estimators(runner, list(CEILING_US), d, w, 100)
    del runner
    torch.cuda.empty_cache()
    slow = {n: round(per[n]["us_per_launch"], 2) for n in CEILING_US if per[n]["us_per_launch"] > CEILING_US[n]}
    assert not slow, "slower than the ceiling (us): %s" % slow


# bfloat16 storage, same workload and method; 1.5x above the current kernels
# (discounted returns 10.8 us, TD(lambda) / GAE 10.3 us, V-trace 14.8 us,
# Retrace 15.5 us, traces / prefix sums 8.4 us), which include the one-item
# routing of the 16-bit formats.
CEILING_BF16_US = {
    "discounted_returns": 16.5,
    "td_lambda": 15.5,
    "gae": 15.5,
    "vtrace": 22.0,
    "retrace": 23.5,
    "eligibility_traces": 12.5,
    "episodic_prefix_sum": 12.5,
}


def test_per_estimator_time_at_16384x256_bfloat16():
    import torch
    import bench
    from linear_recurrence_scan_reverse_amd import synth
    w = synth.WORKLOADS["all7_16384x256"]
    d = synth.workload_inputs(w)
    runner = bench.Runner(w, d, 9, torch.device("cuda", 0), storage="bf16")
    per = bench.time_estimators(runner, list(CEILING_BF16_US), d, w, 100)
    del runner
    torch.cuda.empty_cache()
    slow = {n: round(per[n]["us_per_launch"], 2) for n in CEILING_BF16_US
            if per[n]["us_per_launch"] > CEILING_BF16_US[n]}
    assert not slow, "slower than the ceiling (us): %s" % slow
