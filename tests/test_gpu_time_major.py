"""Time-major [T, E] layout of the seven estimators against the oracle.

The oracle runs on the [E, T] arrays; the kernel gets the same arrays
transposed to [T, E] (flags and trunc_bootstrap included, bootstrap_value /
init stay [E]) and its [T, E] outputs are transposed back before comparing.
Every storage format runs: float32 within the 1e-5 gate, the 16-bit formats
to the rule of ``estimators.check_storage``.  Shapes: one step, one env,
environment counts around the 64-lane block (63, 64, 65, 130), ragged and
whole super-tiles, several super-tiles per column, optional inputs absent,
dense flags, and bases one element off alignment.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from linear_recurrence_scan_reverse_amd import synth
from tests.estimators import TOL, check_storage, parity_err

pytestmark = pytest.mark.gpu

# the seven estimators and the two-output pass
SEVEN = ("discounted_returns", "td_lambda", "gae", "vtrace", "retrace", "eligibility_traces",
         "episodic_prefix_sum", "returns_and_td_lambda")
FORMATS = ("float32", "bfloat16", "float16")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("E,T", [(1, 1), (1, 300), (5, 1), (63, 17), (64, 128), (65, 129), (130, 256),
                                 (1000, 300), (200, 1000)])
def test_time_major_all_estimators(fmt, E, T):
    _say("time-major %s E=%d T=%d" % (fmt, E, T))
    d = synth.draw(E, T, seed=80 + E, p_term=0.01, p_trunc=0.01)
    for name in SEVEN:
        check_storage(name, d, fmt, time_major=True)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("variant", [dict(term=False, trunc=False), dict(boot=False, tboot=False),
                                     dict(trunc=False), dict(tboot=False)])
def test_time_major_optional_inputs(fmt, variant):
    d = synth.draw(96, 200, seed=81, p_term=0.02, p_trunc=0.02)
    for name in SEVEN:
        check_storage(name, d, fmt, time_major=True, **variant)


@pytest.mark.parametrize("fmt", FORMATS)
def test_time_major_dense_flags_and_misaligned(fmt):
    d = synth.draw(70, 150, seed=82, p_term=0.2, p_trunc=0.2)
    for name in SEVEN:
        check_storage(name, d, fmt, time_major=True)
        check_storage(name, d, fmt, time_major=True, misalign=True)


def test_time_major_matches_row_major_fp32():
    # both layouts compute the same function: float32 outputs agree within the gate
    import torch
    from tests.estimators import run_gpu, storage_inputs
    d = synth.draw(512, 256, seed=83, p_term=0.01, p_trunc=0.01)
    _, rm = storage_inputs(d)
    _, tm = storage_inputs(d, time_major=True)
    for name in SEVEN:
        a = run_gpu(name, rm)
        b = run_gpu(name, tm, time_major=True)
        torch.cuda.synchronize()
        for k in a:
            err = parity_err(b[k].t().cpu().numpy(), a[k].cpu().numpy().astype(np.float64))
            assert err <= TOL, (name, k, err)


def test_time_major_bitwise_deterministic():
    import torch
    from tests.estimators import run_gpu, storage_inputs
    d = synth.draw(300, 333, seed=84, p_term=0.01, p_trunc=0.01)
    _, tm = storage_inputs(d, time_major=True)
    for name in SEVEN:
        a = {k: v.cpu().numpy() for k, v in run_gpu(name, tm, time_major=True).items()}
        b = {k: v.cpu().numpy() for k, v in run_gpu(name, tm, time_major=True).items()}
        torch.cuda.synchronize()
        for k in a:
            assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), (name, k)


def test_time_major_exact_integer_sums():
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    import oracle
    rng = np.random.default_rng(85)
    E, T = 200, 500
    x = rng.integers(-20, 21, size=(E, T)).astype(np.float32)
    term = (rng.random((E, T)) < 0.01).astype(np.uint8)
    init = rng.integers(-5, 6, size=E).astype(np.float32)
    ref = oracle.episodic_prefix_sum(x, term, None, init)
    got = rl.episodic_prefix_sum(torch.from_numpy(x.T.copy()).cuda(), torch.from_numpy(term.T.copy()).cuda(),
                                 None, torch.from_numpy(init).cuda(), time_major=True)
    assert tuple(got.shape) == (T, E)
    assert np.array_equal(got.cpu().numpy().T.astype(np.float64), ref)


# The item form of float32 time-major calls (chunks of 64 steps x 64 or 32
# environments staged in LDS and scanned as rows; whole chunks, 16-byte
# aligned arrays, one launch): one chunk, odd and even chunk counts, blocks of
# 32 environments (fewer than 16384; 96 is no multiple of 64) and of 64
# (16384 at 64, 256, 384 and 512 steps, from 256 steps the loads moved by
# DMA, float32 V-trace's flags through registers), 4096 x 1088 (columns of 17 chunks, taken since the blocks are half
# as many as the CUs); dense flags; no episode ends (every row's carry
# crosses every chunk).
@pytest.mark.parametrize("E,T", [(64, 64), (96, 128), (128, 192), (192, 448), (256, 320), (1024, 128), (4096, 256),
                                 (4096, 1088), (16384, 64), (16384, 256), (16384, 384), (16384, 512)])
@pytest.mark.parametrize("p", [0.0, 0.01, 0.3])
def test_time_major_item_form(E, T, p):
    if p != 0.01 and E * T > (1 << 20):
        pytest.skip("flag densities are covered at the smaller shapes")
    _say("time-major item form E=%d T=%d p=%g" % (E, T, p))
    d = synth.draw(E, T, seed=89 + E + T, p_term=p, p_trunc=p)
    for name in SEVEN:
        check_storage(name, d, "float32", time_major=True)


# The item form with 16-bit storage (values widened on the way into LDS and
# rounded to nearest even on the way out): both block sizes, one and several
# chunks, dense flags, and 16384 x 256 (the item form for discounted returns,
# TD(lambda) and GAE there, the other kernel for the rest).
@pytest.mark.parametrize("fmt", ("bfloat16", "float16"))
@pytest.mark.parametrize("E,T,p", [(64, 64, 0.01), (96, 128, 0.3), (256, 320, 0.01), (4096, 256, 0.01),
                                   (16384, 256, 0.01), (16384, 384, 0.01)])
def test_time_major_item_form_16bit(fmt, E, T, p):
    _say("time-major item form %s E=%d T=%d p=%g" % (fmt, E, T, p))
    d = synth.draw(E, T, seed=91 + E + T, p_term=p, p_trunc=p)
    for name in SEVEN:
        check_storage(name, d, fmt, time_major=True)


# The DMA form of 64-environment blocks (from 16384 environments, columns of
# at least 256 steps): dense and absent flags, even and odd chunk counts,
# 16-bit storage, and the optional inputs left out (without flags V-trace's
# three streams fit it too).
@pytest.mark.parametrize("fmt", ("float32", "bfloat16", "float16"))
@pytest.mark.parametrize("T,p", [(256, 0.3), (320, 0.0), (320, 0.3)])
def test_time_major_dma_form(fmt, T, p):
    _say("time-major DMA form %s E=16384 T=%d p=%g" % (fmt, T, p))
    d = synth.draw(16384, T, seed=97 + T, p_term=p, p_trunc=p)
    for name in SEVEN:
        check_storage(name, d, fmt, time_major=True)


@pytest.mark.parametrize("fmt", ("float32", "bfloat16"))
@pytest.mark.parametrize("variant", [dict(term=False, trunc=False), dict(boot=False, tboot=False),
                                     dict(tboot=False)])
def test_time_major_dma_form_optional_inputs(fmt, variant):
    d = synth.draw(16384, 256, seed=98, p_term=0.03, p_trunc=0.03)
    for name in SEVEN:
        check_storage(name, d, fmt, time_major=True, **variant)


@pytest.mark.parametrize("variant", [dict(term=False, trunc=False), dict(boot=False, tboot=False),
                                     dict(trunc=False), dict(term=False), dict(tboot=False)])
def test_time_major_item_form_optional_inputs(variant):
    d = synth.draw(128, 320, seed=90, p_term=0.03, p_trunc=0.03)
    for name in SEVEN:
        check_storage(name, d, "float32", time_major=True, **variant)


# Few column groups and long columns: time is cut into segments scanned in
# three launches (segment maps parked in the first output, a carry pass, a
# rescan).  Shapes: two segments, a ragged last segment, two column groups,
# a 512-step segment length with over a hundred segments, many groups with
# few steps each; one environment (laid out like one row, scanned by the
# row-major path, whose long rows are segmented too).
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("E,T", [(2, 512), (3, 4097), (65, 2000), (5, 70000), (130, 8192), (1, 262144)])
def test_time_major_segmented_columns(fmt, E, T):
    _say("time-major segmented %s E=%d T=%d" % (fmt, E, T))
    d = synth.draw(E, T, seed=86 + E, p_term=0.001, p_trunc=0.001)
    for name in SEVEN:
        check_storage(name, d, fmt, time_major=True)


@pytest.mark.parametrize("variant", [dict(term=False, trunc=False), dict(boot=False, tboot=False),
                                     dict(trunc=False), dict(tboot=False)])
def test_time_major_segmented_optional_inputs(variant):
    d = synth.draw(40, 3000, seed=87, p_term=0.002, p_trunc=0.002)
    for name in SEVEN:
        check_storage(name, d, "float32", time_major=True, **variant)
        check_storage(name, d, "bfloat16", time_major=True, misalign=True, **variant)


def test_time_major_segmented_no_cuts_and_deterministic():
    # no episode ends: every segment's carry crosses into the next one
    import torch
    from tests.estimators import run_gpu, storage_inputs
    d = synth.draw(7, 20000, seed=88, p_term=0.0, p_trunc=0.0)
    for name in SEVEN:
        check_storage(name, d, "float32", time_major=True)
    _, tm = storage_inputs(d, time_major=True)
    for name in SEVEN:
        a = {k: v.cpu().numpy() for k, v in run_gpu(name, tm, time_major=True).items()}
        b = {k: v.cpu().numpy() for k, v in run_gpu(name, tm, time_major=True).items()}
        torch.cuda.synchronize()
        for k in a:
            assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), (name, k)
