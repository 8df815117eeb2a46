"""The kernels whose items are 1 KiB of every array (rows of 64, 128 or 256
float32 steps; two items per wave with the second staged through LDS or held
in registers, or four items per wave in registers) against the oracle, at
shapes the launcher routes to each form: discounted returns at every E;
TD(lambda) and GAE everywhere (four per wave at 16384-32767 rows of 256
steps); V-trace four per wave at 16384-32767 rows of 128 or 256 steps and
from 65536 rows of 64, two in registers at 32768 x 64, from 65536 rows of
128 and from 4096 rows of 256, LDS from 32768 rows of 256; Retrace in
registers up to 32767 rows of 64 and up to 4096 rows, four per wave from
32768 rows of 64 and at 16384-65535 rows of 128, LDS at 4097-32768 rows of
256 (four of item B's five streams in LDS up to 16384 rows, three above) and
from 65536 rows of 128; traces and prefix sums LDS for rows of 64 up
to 16384 rows and from 65536 rows of 256, registers up to 4096 rows, at
16384 x 128 and 32768 x 64.  Row counts that leave the last block with waves
that have fewer items, or the last item with fewer than 64 / L rows, are
included, as are absent optional inputs.  The 16-bit formats' register form
is covered in test_gpu_storage16.py."""
from __future__ import annotations

import sys

import pytest

from linear_recurrence_scan_reverse_amd import synth
from tests.estimators import TOL, compare

pytestmark = pytest.mark.gpu

CASES = (
    [("discounted_returns", E, T) for (E, T) in [(1, 64), (3, 64), (13, 64), (5, 128), (9, 256), (1000, 128),
                                                 (1001, 256), (4099, 64), (16385, 256)]]
    + [("retrace", E, T) for (E, T) in [(3, 64), (1001, 128), (4096, 128), (9, 256), (9001, 256), (16384, 256),
                                        (16385, 256), (16387, 128), (32769, 64), (65536, 128)]]
    + [("vtrace", E, T) for (E, T) in [(4096, 256), (4099, 256), (20001, 256), (65537, 128), (16385, 128),
                                       (32768, 64), (65537, 64), (32769, 256)]]
    + [(n, E, T) for n in ("td_lambda", "gae") for (E, T) in [(7, 64), (1001, 128), (4096, 256), (16385, 256),
                                                                 (32768, 256), (32771, 256), (65536, 128)]]
    + [(n, E, T) for n in ("eligibility_traces", "episodic_prefix_sum")
       for (E, T) in [(5, 64), (1001, 128), (4096, 256), (16383, 64), (16384, 128), (32768, 64), (65537, 256)]]
)


@pytest.mark.parametrize("name,E,T", CASES)
def test_duo_kernel_matches_oracle(name, E, T):
    print("duo %s E=%d T=%d" % (name, E, T), file=sys.stderr, flush=True)
    d = synth.draw(E, T, seed=90 + E % 13, p_term=0.01, p_trunc=0.01)
    for k, (err, mx) in compare(name, d).items():
        assert err <= TOL, "%s %s E=%d T=%d: err %.3g (max|ref| %.3g)" % (name, k, E, T, err, mx)


@pytest.mark.parametrize("variant", [dict(term=False, trunc=False), dict(boot=False, tboot=False), dict(trunc=False),
                                     dict(tboot=False)])
@pytest.mark.parametrize("name", ["discounted_returns", "vtrace", "retrace"])
def test_duo_kernel_optional_inputs(name, variant):
    d = synth.draw(4101, 256, seed=97, p_term=0.02, p_trunc=0.02)
    for k, (err, mx) in compare(name, d, **variant).items():
        assert err <= TOL, "%s %s %s: err %.3g" % (name, variant, k, err)


def test_duo_kernel_dense_flags_and_exact_sums():
    import numpy as np
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    import oracle
    d = synth.draw(33001, 256, seed=98, p_term=0.3, p_trunc=0.3)
    for name in ("discounted_returns", "td_lambda", "eligibility_traces"):
        for k, (err, mx) in compare(name, d).items():
            assert err <= TOL, (name, k, err)
    # small-integer prefix sums are exact on this path too
    rng = np.random.default_rng(99)
    x = rng.integers(-20, 21, size=(32768, 256)).astype(np.float32)
    term = (rng.random((32768, 256)) < 0.01).astype(np.uint8)
    got = rl.episodic_prefix_sum(torch.from_numpy(x).cuda(), torch.from_numpy(term).cuda()).cpu().numpy()
    assert np.array_equal(got.astype(np.float64), oracle.episodic_prefix_sum(x, term))
