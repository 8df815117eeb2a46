"""Vector-valued eligibility traces ([E, T, D] features) against the oracle."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from linear_recurrence_scan_reverse_amd import synth
from tests.estimators import TOL, parity_err

pytestmark = pytest.mark.gpu


def _run(f, with_flags=True, with_init=True, gamma=0.99, lam=0.95):
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in f.items()}
    got = rl.eligibility_traces_vec(dev["x"], dev["terminated"] if with_flags else None,
                                    dev["truncated"] if with_flags else None,
                                    dev["init"] if with_init else None, gamma=gamma, lam=lam)
    ref = oracle.eligibility_traces_vec(f["x"], f["terminated"] if with_flags else None,
                                        f["truncated"] if with_flags else None,
                                        f["init"] if with_init else None, gamma=gamma, lam=lam)
    return got.cpu().numpy(), ref


@pytest.mark.parametrize("E,T,D", [(1, 1, 1), (3, 7, 5), (5, 256, 64), (2, 1000, 3), (64, 128, 130),
                                   (17, 33, 1), (1, 9, 200)])
def test_vector_traces_parity(E, T, D):
    f = synth.draw_features(E, T, D, seed=70 + T + D, p_term=0.03, p_trunc=0.03)
    for flags in (True, False):
        for init in (True, False):
            got, ref = _run(f, flags, init)
            assert parity_err(got, ref) <= TOL, (E, T, D, flags, init)


@pytest.mark.parametrize("gamma,lam", [(0.0, 0.0), (1.0, 1.0), (0.5, 0.9)])
def test_vector_traces_parameters_and_dense_flags(gamma, lam):
    f = synth.draw_features(9, 300, 40, seed=71, p_term=0.3, p_trunc=0.3)
    got, ref = _run(f, gamma=gamma, lam=lam)
    assert parity_err(got, ref) <= TOL


def test_vector_traces_full_size_and_deterministic():
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    f = synth.draw_features(1024, 256, 64, seed=0, p_term=0.004, p_trunc=0.004)
    got, ref = _run(f)
    assert parity_err(got, ref) <= TOL
    dev = {k: torch.from_numpy(v).cuda() for k, v in f.items()}
    a = rl.eligibility_traces_vec(dev["x"], dev["terminated"], dev["truncated"], dev["init"])
    b = rl.eligibility_traces_vec(dev["x"], dev["terminated"], dev["truncated"], dev["init"])
    assert torch.equal(a, b)


@pytest.mark.parametrize("fmt", ["float32", "bfloat16", "float16"])
@pytest.mark.parametrize("time_major", [False, True])
@pytest.mark.parametrize("E,T,D", [(1, 1, 1), (3, 7, 5), (5, 256, 64), (17, 33, 70), (64, 100, 3)])
def test_vector_traces_formats_and_layouts(fmt, time_major, E, T, D):
    # values rounded to the format (the oracle runs on them, widened); time-major
    # takes x as [T, E, D] and flags as [T, E]
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    from tests.estimators import check_rounded
    dt = getattr(torch, fmt)
    f = synth.draw_features(E, T, D, seed=80 + T + D, p_term=0.03, p_trunc=0.03)
    x = torch.from_numpy(f["x"]).to(dt)
    init = torch.from_numpy(f["init"]).to(dt)
    hx, hi = x.float().numpy(), init.float().numpy()
    te, tr = (torch.from_numpy(f[k]) for k in ("terminated", "truncated"))
    if time_major:
        xd, ted, trd = x.transpose(0, 1).contiguous(), te.t().contiguous(), tr.t().contiguous()
    else:
        xd, ted, trd = x, te, tr
    got = rl.eligibility_traces_vec(xd.cuda(), ted.cuda(), trd.cuda(), init.cuda(), gamma=0.99, lam=0.95,
                                    time_major=time_major)
    torch.cuda.synchronize()
    if time_major:
        got = got.transpose(0, 1).contiguous()
    ref = oracle.eligibility_traces_vec(hx, f["terminated"], f["truncated"], hi, gamma=0.99, lam=0.95)
    check_rounded(got, ref, fmt, "traces_vec %s tm=%s E=%d T=%d D=%d" % (fmt, time_major, E, T, D))
