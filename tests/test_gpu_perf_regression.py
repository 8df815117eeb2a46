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


# Time-major float32 arrays, same method; 1.2x above the current kernels at
# 16384 x 256 (discounted returns 11.3 us, TD(lambda) / GAE 13.9 us, V-trace
# 21.1 us, Retrace 24.8 us, traces / prefix sums 9.6 us), at 4096 x 512
# (discounted returns 12.8 us, TD(lambda) 14.3 us, V-trace 18.9 us, Retrace
# 20.6 us, traces 9.0 us; the segmented path took 24-42 us there) and at
# 32768 x 64 (discounted returns 7.9 us, TD(lambda) 10.8 us, V-trace 15.3 us,
# traces 6.6 us; 15-21 us before the item form).
CEILING_TM_US = {
    (16384, 256): {"discounted_returns": 13.6, "td_lambda": 16.7, "gae": 16.7, "vtrace": 25.4, "retrace": 29.8,
                   "eligibility_traces": 11.5, "episodic_prefix_sum": 11.5},
    (4096, 512): {"discounted_returns": 15.4, "td_lambda": 17.2, "vtrace": 22.7, "retrace": 24.7,
                  "eligibility_traces": 10.8},
    (32768, 64): {"discounted_returns": 9.5, "td_lambda": 13.0, "vtrace": 18.4, "eligibility_traces": 7.9},
}


@pytest.mark.parametrize("E,T", list(CEILING_TM_US))
def test_per_estimator_time_major(E, T):
    import dataclasses
    import torch
    import bench
    from linear_recurrence_scan_reverse_amd import synth
    ceiling = CEILING_TM_US[(E, T)]
    w = dataclasses.replace(synth.WORKLOADS["all7_16384x256"], name="all7_%dx%d" % (E, T), E=E, T=T)
    d = synth.workload_inputs(w)
    set_bytes = E * T * (4 * 8 + 2 + 4 * 8) + 4 * E
    runner = bench.Runner(w, d, int(min(64, max(2, -(-(1 << 30) // set_bytes) + 1))), torch.device("cuda", 0),
                          time_major=True)
    per = bench.time_estimators(runner, list(ceiling), d, w, 200)
    del runner
    torch.cuda.empty_cache()
    slow = {n: round(per[n]["us_per_launch"], 2) for n in ceiling if per[n]["us_per_launch"] > ceiling[n]}
    assert not slow, "slower than the ceiling (us): %s" % slow
