"""Seeded random configurations against the oracle.

Each case draws an estimator (the seven and the two-output pass), a storage
format, a layout, a shape (E up to 600, T up to 700, log-uniform), flag rates
(0 to 0.5), which optional inputs are passed, and the parameters (gamma and
lambda anywhere in [0, 1], ends included; V-trace clips in (0, 2]), and checks
the GPU result with ``estimators.check_storage``.  The draws come from one
numpy generator per case, so a failure names a reproducible case.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from linear_recurrence_scan_reverse_amd import synth
from tests.estimators import NAMES, check_storage

pytestmark = pytest.mark.gpu

N_CASES = 160


def _case(i):
    rng = np.random.default_rng(1000 + i)
    name = NAMES[rng.integers(len(NAMES))]
    fmt = ("float32", "bfloat16", "float16")[rng.integers(3)]
    tm = bool(rng.integers(2))
    E = int(np.exp(rng.uniform(0, np.log(600))))
    T = int(np.exp(rng.uniform(0, np.log(700))))
    p = [0.0, 0.001, 0.05, 0.5]
    pt, pr = p[rng.integers(4)], p[rng.integers(4)]
    variant = dict(term=bool(rng.integers(4)), trunc=bool(rng.integers(4)), boot=bool(rng.integers(3)),
                   tboot=bool(rng.integers(3)))
    ends = [0.0, 1.0]
    g = ends[rng.integers(2)] if rng.random() < 0.2 else float(rng.uniform(0, 1))
    lam = ends[rng.integers(2)] if rng.random() < 0.2 else float(rng.uniform(0, 1))
    P = dict(gamma=g, lam=lam, vtrace_lam=float(rng.uniform(0, 1)), rho_bar=float(rng.uniform(0.05, 2)),
             c_bar=float(rng.uniform(0.05, 2)))
    return name, fmt, tm, E, T, pt, pr, variant, P, int(rng.integers(1 << 30))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    name, fmt, tm, E, T, pt, pr, variant, P, seed = _case(i)
    print("case %d: %s %s tm=%s E=%d T=%d p=(%g, %g) %s %s" % (i, name, fmt, tm, E, T, pt, pr, variant, P),
          file=sys.stderr, flush=True)
    d = synth.draw(E, T, seed=seed, p_term=pt, p_trunc=pr)
    check_storage(name, d, fmt, time_major=tm, P=P, **variant)
