"""Long rows with few rows: the segmented path against the oracle.

Rows of 16384 steps or more, with at most 64 rows, are cut into segments
scanned by separate waves in three passes: segment maps, a per-row scan over
the segment maps, and a rescan of every segment from its entering value.
These tests cover ragged and whole-tile rows, one to 64 rows (and 65, just past the limit),
sparse and dense flags, NULL optional inputs, the generic recurrence with a
carry, exact integer sums across segments and run-to-run determinism.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from linear_recurrence_scan_reverse_amd import synth
from tests.estimators import NAMES, TOL, compare, parity_err, to_dev

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _check(name, d, what, **variant):
    res = compare(name, d, **variant)
    for k, (e, mx) in res.items():
        assert e <= TOL, "%s %s %s: err %.3g (max|ref| %.3g)" % (name, k, what, e, mx)
    return max(e for e, _ in res.values())


@pytest.mark.parametrize("E,T", [(1, 16384), (3, 20000), (2, 65536), (17, 50021), (64, 16640), (65, 16640), (1, 1 << 20)])
def test_long_rows_all_estimators(E, T):
    _say("long rows E=%d T=%d" % (E, T))
    d = synth.draw(E, T, seed=40 + E, p_term=0.0005, p_trunc=0.0005)
    for name in NAMES:
        _check(name, d, "E=%d T=%d" % (E, T))


@pytest.mark.parametrize("variant", [dict(term=False, trunc=False), dict(boot=False, tboot=False),
                                     dict(trunc=False), dict(tboot=False)])
def test_long_rows_optional_inputs(variant):
    d = synth.draw(3, 40000, seed=41, p_term=0.002, p_trunc=0.002)
    for name in NAMES:
        _check(name, d, str(variant), **variant)


def test_long_rows_dense_flags():
    d = synth.draw(2, 30000, seed=42, p_term=0.05, p_trunc=0.05)
    for name in NAMES:
        _check(name, d, "dense flags")


def test_long_rows_generic_scan_and_exact_sums():
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    import oracle
    rng = np.random.default_rng(43)
    E, T = 3, 70001
    a = rng.uniform(-1.0, 1.0, size=(E, T)).astype(np.float32)
    b = rng.standard_normal((E, T)).astype(np.float32)
    c = rng.standard_normal(E).astype(np.float32)
    ad, bd, cd = (torch.from_numpy(v).cuda() for v in (a, b, c))
    for rev in (True, False):
        got = rl.linear_scan(ad, bd, cd, reverse=rev).cpu().numpy()
        assert parity_err(got, oracle.linear_scan(a, b, c, reverse=rev)) <= TOL
    # a = 1 and small integers: suffix / prefix sums across every segment edge are exact
    ones = np.ones((E, T), dtype=np.float32)
    bi = rng.integers(-3, 4, size=(E, T)).astype(np.float32)
    ci = rng.integers(-100, 101, size=E).astype(np.float32)
    for rev in (True, False):
        got = rl.linear_scan(torch.from_numpy(ones).cuda(), torch.from_numpy(bi).cuda(),
                             torch.from_numpy(ci).cuda(), reverse=rev).cpu().numpy()
        assert np.array_equal(got.astype(np.float64), oracle.linear_scan(ones, bi, ci, reverse=rev))
    x = rng.integers(-20, 21, size=(E, T)).astype(np.float32)
    term = (rng.random((E, T)) < 0.0003).astype(np.uint8)
    got = rl.episodic_prefix_sum(torch.from_numpy(x).cuda(), torch.from_numpy(term).cuda()).cpu().numpy()
    assert np.array_equal(got.astype(np.float64), oracle.episodic_prefix_sum(x, term))


def test_long_rows_bitwise_deterministic():
    import torch
    from tests.estimators import run_gpu
    d = synth.draw(5, 33000, seed=44, p_term=0.001, p_trunc=0.001)
    dd = to_dev(d)
    for name in NAMES:
        a = {k: v.cpu().numpy() for k, v in run_gpu(name, dd).items()}
        b = {k: v.cpu().numpy() for k, v in run_gpu(name, dd).items()}
        torch.cuda.synchronize()
        for k in a:
            assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), (name, k)


# Rows whose length is a whole number of segments plus 1..7 steps: the last
# segment takes the remainder, so its parked float64 pair (4 float32 or 8
# 16-bit elements) stays inside it.  The first output sits at the start of a
# larger buffer whose tail holds a sentinel that must survive the call.
RAGGED = [(E, T) for E in (1, 2, 64) for T in (16385, 16387, 17409)]


def _guarded(E, T, dtype):
    import torch
    guard = 64
    buf = torch.full((E * T + guard,), -7.25, dtype=dtype, device="cuda")
    return buf, buf[:E * T].view(E, T), guard


def _guard_intact(buf, n, label):
    import torch
    tail = buf[n:].float().cpu()
    assert torch.all(tail == -7.25), "%s: wrote past the end of the first output" % label


@pytest.mark.parametrize("fmt", ["float32", "bfloat16"])
@pytest.mark.parametrize("E,T", RAGGED + [(E, 16391) for E in (1, 2, 64)])
def test_ragged_last_segment(fmt, E, T):
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    import oracle
    from tests.estimators import check_rounded, run_gpu, run_oracle, storage_inputs
    _say("ragged last segment %s E=%d T=%d" % (fmt, E, T))
    dt = getattr(torch, fmt)
    d = synth.draw(E, T, seed=45 + T % 97, p_term=0.001, p_trunc=0.001)
    host, dev = storage_inputs(d, fmt)
    for name in NAMES:
        buf, out0, _ = _guarded(E, T, dt)
        got = run_gpu(name, dev, out0=out0)
        torch.cuda.synchronize()
        ref = run_oracle(name, host)
        label = "%s %s E=%d T=%d" % (name, fmt, E, T)
        for k, r in ref.items():
            check_rounded(got[k], r, fmt, label + " " + k)
        _guard_intact(buf, E * T, label)
    # the generic recurrence, both directions, without and with episode cuts
    rng = np.random.default_rng(46)
    a = rng.uniform(-1.0, 1.0, size=(E, T)).astype(np.float32)
    b = rng.standard_normal((E, T)).astype(np.float32)
    c = rng.standard_normal(E).astype(np.float32)
    done = (rng.random((E, T)) < 0.001).astype(np.uint8)
    ta, tb, tc = (torch.from_numpy(v).to(dt) for v in (a, b, c))
    ha, hb, hc = (t.float().numpy() for t in (ta, tb, tc))
    for rev in (True, False):
        for cut in (None, done):
            buf, out0, _ = _guarded(E, T, dt)
            rl.linear_scan_segmented(ta.cuda(), tb.cuda(), None if cut is None else torch.from_numpy(cut).cuda(),
                                     tc.cuda(), reverse=rev, out=out0)
            torch.cuda.synchronize()
            label = "linear scan %s rev=%s cuts=%s E=%d T=%d" % (fmt, rev, cut is not None, E, T)
            check_rounded(out0, oracle.linear_scan_segmented(ha, hb, cut, hc, reverse=rev), fmt, label)
            _guard_intact(buf, E * T, label)
