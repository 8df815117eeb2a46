"""The generic recurrence (with and without episode cuts) in every storage
format and both layouts, against the oracle.

a ~ U(-0.95, 0.95), b ~ N(0, 1), carry ~ N(0, 1) and done ~ B(p) are drawn in
float32, rounded to the format, and the oracle runs on the widened values.
Outputs follow the rule of ``estimators.check_rounded``.  Shapes cover short
rows sharing a wave, whole and ragged tiles, multi-wave rows, long rows on the
segmented path (row-major) and environment counts around the 64-lane
time-major block.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from tests.estimators import check_rounded

pytestmark = pytest.mark.gpu

FORMATS = ("float32", "bfloat16", "float16")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _draw(E, T, seed, p_cut):
    rng = np.random.default_rng(seed)
    a = rng.uniform(-0.95, 0.95, size=(E, T)).astype(np.float32)
    b = rng.standard_normal((E, T)).astype(np.float32)
    c = rng.standard_normal(E).astype(np.float32)
    done = (rng.random((E, T)) < p_cut).astype(np.uint8) if p_cut > 0 else None
    return a, b, c, done


def _run(fmt, E, T, seed, p_cut, time_major, with_carry=True):
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    dt = getattr(torch, fmt)
    a, b, c, done = _draw(E, T, seed, p_cut)
    ta, tb, tc = (torch.from_numpy(x).to(dt) for x in (a, b, c))
    ha, hb, hc = (x.float().numpy() for x in (ta, tb, tc))
    def dev(x):
        return (x.t().contiguous() if time_major else x).cuda()
    td = torch.from_numpy(done) if done is not None else None
    for rev in (True, False):
        got = rl.linear_scan_segmented(dev(ta), dev(tb), dev(td) if td is not None else None,
                                       tc.cuda() if with_carry else None, reverse=rev, time_major=time_major)
        torch.cuda.synchronize()
        if time_major:
            got = got.t().contiguous()
        ref = oracle.linear_scan_segmented(ha, hb, done, hc if with_carry else None, reverse=rev)
        check_rounded(got, ref, fmt, "%s E=%d T=%d tm=%s rev=%s cut=%g" % (fmt, E, T, time_major, rev, p_cut))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("E,T", [(1, 1), (3, 5), (256, 128), (100, 256), (37, 1000), (64, 1024), (130, 300)])
@pytest.mark.parametrize("p_cut", [0.0, 0.02])
def test_generic_scan_formats(fmt, E, T, p_cut):
    _run(fmt, E, T, 100 + T, p_cut, time_major=False)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("E,T", [(1, 1), (63, 17), (64, 128), (65, 257), (1000, 300), (4, 5000), (70, 3000)])
@pytest.mark.parametrize("p_cut", [0.0, 0.02])
def test_generic_scan_time_major(fmt, E, T, p_cut):
    _run(fmt, E, T, 200 + E, p_cut, time_major=True)


@pytest.mark.parametrize("fmt", ["bfloat16", "float16"])
def test_generic_scan_16bit_long_rows(fmt):
    _say("generic scan long rows %s" % fmt)
    _run(fmt, 3, 40001, 300, 0.001, time_major=False)
    _run(fmt, 2, 20000, 301, 0.0, time_major=False, with_carry=False)


def test_generic_scan_exact_sums_every_format():
    # a = 1, small integer b and carry: suffix / prefix sums below 256 are exact
    # in every format and both layouts
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    rng = np.random.default_rng(302)
    E, T = 96, 200
    a = np.ones((E, T), dtype=np.float32)
    b = rng.integers(-1, 2, size=(E, T)).astype(np.float32)
    c = rng.integers(-3, 4, size=E).astype(np.float32)
    done = (rng.random((E, T)) < 0.05).astype(np.uint8)
    for fmt in FORMATS:
        dt = getattr(torch, fmt)
        for tm in (False, True):
            for rev in (True, False):
                ref = oracle.linear_scan_segmented(a, b, done, c, reverse=rev)
                assert np.max(np.abs(ref)) < 256
                f = (lambda x: torch.from_numpy(x.T.copy() if tm else x).cuda())
                got = rl.linear_scan_segmented(f(a).to(dt), f(b).to(dt), f(done), torch.from_numpy(c).to(dt).cuda(),
                                               reverse=rev, time_major=tm)
                got = got.float().cpu().numpy()
                got = got.T if tm else got
                assert np.array_equal(got.astype(np.float64), ref), (fmt, tm, rev)
