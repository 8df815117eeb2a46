"""16-bit storage (bfloat16, float16) of the seven estimators against the oracle.

The inputs are drawn in float32, rounded to the storage format, and the
oracle runs in float64 on exactly the values the kernel reads (the 16-bit
values widened).  The kernel rounds each float64 result to float32 and then
to the format, both to nearest even, so (``estimators.check_storage``):

* every output is within the format's unit roundoff u of the exact value
  (u = 2^-8 for bfloat16, 2^-11 for float16; relative where |ref| >= 1,
  absolute below), plus the 1e-5 float32 gate;
* almost every output is bit-equal to the oracle's value rounded the same
  way; the rest (a float64 result within a few ulps of a rounding midpoint)
  differ by one unit in the last place.

Shapes cover the streaming kernel (traces and prefix sums; whole tiles,
16-byte aligned, E even), the pipelined kernel's vector path and element path
(ragged rows, odd E, arrays whose base is only 2-byte aligned), short rows
sharing a wave, multi-wave rows, long rows on the segmented path and absent
optional inputs.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from linear_recurrence_scan_reverse_amd import synth
from tests.estimators import check_storage

pytestmark = pytest.mark.gpu

# the seven estimators and the two-output pass
SEVEN = ("discounted_returns", "td_lambda", "gae", "vtrace", "retrace", "eligibility_traces",
         "episodic_prefix_sum", "returns_and_td_lambda")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("fmt", ["bfloat16", "float16"])
@pytest.mark.parametrize("E,T", [(1, 1), (3, 5), (256, 128), (100, 256), (37, 1000), (64, 1024), (513, 300),
                                 (64, 64), (33, 256), (2000, 256), (1000, 128), (998, 64)])
def test_storage16_all_estimators(fmt, E, T):
    _say("16-bit storage %s E=%d T=%d" % (fmt, E, T))
    d = synth.draw(E, T, seed=70 + T, p_term=0.01, p_trunc=0.01)
    for name in SEVEN:
        check_storage(name, d, fmt)


@pytest.mark.parametrize("fmt", ["bfloat16", "float16"])
@pytest.mark.parametrize("variant", [dict(term=False, trunc=False), dict(boot=False, tboot=False),
                                     dict(trunc=False), dict(tboot=False)])
def test_storage16_optional_inputs(fmt, variant):
    d = synth.draw(48, 512, seed=71, p_term=0.02, p_trunc=0.02)
    for name in SEVEN:
        check_storage(name, d, fmt, **variant)


@pytest.mark.parametrize("fmt", ["bfloat16", "float16"])
def test_storage16_two_byte_aligned_bases(fmt):
    # whole tiles, but every array starts one element past an aligned
    # boundary: the element-wise load path runs
    d = synth.draw(64, 256, seed=72, p_term=0.01, p_trunc=0.01)
    for name in SEVEN:
        check_storage(name, d, fmt, misalign=True)


@pytest.mark.parametrize("fmt", ["bfloat16", "float16"])
@pytest.mark.parametrize("E,T", [(2, 40000), (1, 65536)])
def test_storage16_long_rows(fmt, E, T):
    # rows of 16384 steps or more with few rows take the segmented path, whose
    # intermediate float64 values live in the first output's 16-bit elements
    _say("16-bit storage long rows %s E=%d T=%d" % (fmt, E, T))
    d = synth.draw(E, T, seed=73, p_term=0.001, p_trunc=0.001)
    for name in SEVEN:
        check_storage(name, d, fmt)


@pytest.mark.parametrize("fmt", ["bfloat16", "float16"])
def test_storage16_exact_integer_sums(fmt):
    # small integers and their episodic sums below 256 are exact in both
    # formats: the outputs must equal the oracle bit for bit
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    import oracle
    rng = np.random.default_rng(74)
    E, T = 64, 256
    x = rng.integers(-1, 2, size=(E, T)).astype(np.float32)
    term = (rng.random((E, T)) < 0.05).astype(np.uint8)
    ref = oracle.episodic_prefix_sum(x, term)
    assert np.max(np.abs(ref)) < 256
    dt = getattr(torch, fmt)
    got = rl.episodic_prefix_sum(torch.from_numpy(x).to(dt).cuda(), torch.from_numpy(term).cuda())
    assert got.dtype == dt
    assert np.array_equal(got.float().cpu().numpy().astype(np.float64), ref)


def test_float16_overflow_gives_inf():
    # sums rounded to float16 (nearest even); beyond the largest finite value
    # (65504, rounding threshold 65520) they become +inf, not a wrapped value
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    x = torch.full((2, 64), 2000.0, dtype=torch.float16).cuda()
    got = rl.episodic_prefix_sum(x).float().cpu().numpy()
    ref = np.cumsum(np.full((2, 64), 2000.0), axis=1)
    with np.errstate(over="ignore"):
        exp = ref.astype(np.float32).astype(np.float16).astype(np.float32)
    assert np.isposinf(exp[:, -1]).all() and np.isfinite(exp[:, 31]).all()
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("fmt", ["bfloat16", "float16"])
@pytest.mark.parametrize("E,T", [(1, 512), (5, 128), (9, 256), (1001, 512), (4099, 128), (16385, 256), (1001, 256),
                                 (16385, 64), (32768, 64), (3, 64), (16387, 512)])
def test_storage16_two_items_per_wave(fmt, E, T):
    # rows of 64-512 steps with aligned arrays: the kernel that gives each wave
    # two items held in registers, 16 bytes per lane and array (rows of
    # 128-512 steps) or 8 (rows of 64 from 16384 rows, of 128 up to 4096 rows,
    # of 256 up to 4096 rows for the light estimators), where the launcher
    # routes them there, or four items per wave (rows of 512 from 16384 rows:
    # traces, prefix sums, TD(lambda), GAE); row counts leave the last block
    # with waves that have no second item and the last item with fewer rows
    _say("16-bit storage two items per wave %s E=%d T=%d" % (fmt, E, T))
    d = synth.draw(E, T, seed=74 + E % 7, p_term=0.01, p_trunc=0.01)
    for name in SEVEN:
        check_storage(name, d, fmt)
