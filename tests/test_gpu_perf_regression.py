"""Performance regression guard at the all-seven workload (16384 x 256).

Each estimator's per-launch time, measured as the bench measures it (rotating
buffer sets over 1 GiB, 200 back-to-back calls, HIP events on the launch
stream), must stay under a ceiling set 1.2x above what the current kernels
measure on one MI355X (discounted returns 10.6 us, TD(lambda) / GAE 12.2 us,
V-trace 19.1 us, Retrace 19.9 us, traces / prefix sums 8.7 us).  Times move by
up to about 5% from one GPU to the next; a routing or occupancy mistake has
cost 1.3-2x here.
"""
from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu

CEILING_US = {
    "discounted_returns": 12.7,
    "td_lambda": 14.6,
    "gae": 14.6,
    "vtrace": 22.9,
    "retrace": 23.9,
    "eligibility_traces": 10.4,
    "episodic_prefix_sum": 10.4,
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
# (discounted returns 10.7 us, TD(lambda) / GAE 10.2 us, V-trace 14.6 us,
# Retrace 15.1 us, traces / prefix sums 8.2 us).
CEILING_BF16_US = {
    "discounted_returns": 12.9,
    "td_lambda": 12.3,
    "gae": 12.3,
    "vtrace": 17.5,
    "retrace": 18.1,
    "eligibility_traces": 9.8,
    "episodic_prefix_sum": 9.8,
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
