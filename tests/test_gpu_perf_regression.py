"""Performance regression guard at the all-seven workload (16384 x 256).

Each estimator's per-launch time, measured as the bench measures it (rotating
buffer sets over 1 GiB, 200 back-to-back calls, HIP events on the launch
stream), must stay under a ceiling set 1.2x above what the current kernels
measure on one MI355X (discounted returns 9.4 us, TD(lambda) / GAE 12.1 us,
V-trace 19.0 us, Retrace 19.6 us, traces / prefix sums 8.1 us).  Times move by
up to about 5% from one GPU to the next; a routing or occupancy mistake has
cost 1.3-2x here.
"""
from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu

CEILING_US = {
    "discounted_returns": 11.3,
    "td_lambda": 14.5,
    "gae": 14.5,
    "vtrace": 22.8,
    "retrace": 23.5,
    "eligibility_traces": 9.8,
    "episodic_prefix_sum": 9.8,
}


def test_per_estimator_time_at_16384x256():
    import torch
    import bench
    from linear_recurrence_scan_reverse_amd import synth
    w = synth.WORKLOADS["all7_16384x256"]
    d = synth.workload_inputs(w)
    runner = bench.Runner(w, d, 5, torch.device("cuda", 0))
    per = bench.time_estimators(runner, list(CEILING_US), d, w, 200)
    del runner
    torch.cuda.empty_cache()
    slow = {n: round(per[n]["us_per_launch"], 2) for n in CEILING_US if per[n]["us_per_launch"] > CEILING_US[n]}
    assert not slow, "slower than the ceiling (us): %s" % slow


# bfloat16 storage, same workload and method; 1.2x above the current kernels
# (discounted returns 8.0 us, TD(lambda) / GAE 8.8 us, V-trace 12.4 us,
# Retrace 12.8 us, traces / prefix sums 6.7 us).
CEILING_BF16_US = {
    "discounted_returns": 9.6,
    "td_lambda": 10.6,
    "gae": 10.6,
    "vtrace": 14.9,
    "retrace": 15.4,
    "eligibility_traces": 8.0,
    "episodic_prefix_sum": 8.0,
}


def test_per_estimator_time_at_16384x256_bfloat16():
    import torch
    import bench
    from linear_recurrence_scan_reverse_amd import synth
    w = synth.WORKLOADS["all7_16384x256"]
    d = synth.workload_inputs(w)
    runner = bench.Runner(w, d, 9, torch.device("cuda", 0), storage="bf16")
    per = bench.time_estimators(runner, list(CEILING_BF16_US), d, w, 200)
    del runner
    torch.cuda.empty_cache()
    slow = {n: round(per[n]["us_per_launch"], 2) for n in CEILING_BF16_US
            if per[n]["us_per_launch"] > CEILING_BF16_US[n]}
    assert not slow, "slower than the ceiling (us): %s" % slow
