"""Arrays past 2^31 elements, and the longest row the ABI accepts.

Every kernel addresses rows with a 64-bit base and 32-bit in-row offsets, so
the cases that can go wrong are element indices beyond 2^31 (rows past
2^31 / T) and rows near 2^30 steps.  Inputs are drawn on the GPU (seeded
torch generators; the oracle gets the same values copied back), the full
arrays are scanned, and sampled rows (or, for the 2^30-step rows, sampled
episodes) are checked against the oracle:

* [E, T] with E = 2^23 + 3, T = 256 (2^31 + 768 elements, 8 GiB per float32
  array): discounted returns (streaming kernel), GAE (streaming), Retrace
  (pipelined kernel), rows sampled at the start, around element 2^31 and at
  the end;
* the same shape time-major ([T, E]) for TD(lambda), and [320, 2^23 - 64]
  (the largest shape of the time-major item form);
* two rows of 2^30 - 1 steps (the ABI's longest) on the segmented path,
  checked on whole episodes: a slice that ends with a terminated step
  (backward) or starts right after a done step (forward) does not depend on
  anything outside it.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from tests.estimators import TOL, parity_err

pytestmark = pytest.mark.gpu

E_BIG = (1 << 23) + 3
T_BIG = 256
P_FLAG = 0.004


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _free():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _inputs(shape, seed, names):
    """Seeded device draws: values N(0,1), probabilities U(0.05, 1), flags B(P_FLAG)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = {}
    for n in names:
        if n in ("terminated", "truncated"):
            out[n] = (torch.rand(shape, generator=g, device="cuda") < P_FLAG).to(torch.uint8)
        elif n in ("pi", "mu"):
            out[n] = torch.rand(shape, generator=g, device="cuda") * 0.95 + 0.05
        elif n == "bootstrap_value":
            out[n] = torch.randn(shape[0] if len(shape) == 2 else shape, generator=g, device="cuda")
        else:
            out[n] = torch.randn(shape, generator=g, device="cuda")
    return out


def _sample_rows(E, T):
    first_big = (1 << 31) // T  # first row holding an element index >= 2^31
    rows = [0, 1, E // 2, first_big - 1, first_big, first_big + 1, E - 2, E - 1]
    return sorted(set(r for r in rows if 0 <= r < E))


def _rows(t, rows, time_major=False):
    import torch
    idx = torch.tensor(rows, device=t.device)
    if t.dim() == 1:
        return t[idx].cpu().numpy()
    sel = t[:, idx].t() if time_major else t[idx]
    return sel.contiguous().cpu().numpy()


@pytest.mark.parametrize("name", ["discounted_returns", "gae", "retrace"])
def test_rows_past_2pow31_elements(name):
    import linear_recurrence_scan_reverse_amd as rl
    E, T = E_BIG, T_BIG
    _say("max sizes %s E=%d T=%d" % (name, E, T))
    need = {"discounted_returns": ["r"], "gae": ["r", "v"], "retrace": ["r", "q", "exp_q", "pi", "mu"]}[name]
    d = _inputs((E, T), 90, need + ["bootstrap_value", "trunc_bootstrap", "terminated", "truncated"])
    fl = (d["terminated"], d["truncated"], d["bootstrap_value"], d["trunc_bootstrap"])
    if name == "discounted_returns":
        out = {"out": rl.discounted_returns(d["r"], *fl, gamma=0.99)}
    elif name == "gae":
        adv, ret = rl.gae(d["r"], d["v"], *fl, gamma=0.99, lam=0.95, with_returns=True)
        out = {"out": adv, "out1": ret}
    else:
        out = {"out": rl.retrace(d["r"], d["q"], d["exp_q"], d["pi"], d["mu"], *fl, gamma=0.99, lam=0.95)}
    rows = _sample_rows(E, T)
    h = {k: _rows(v, rows) for k, v in d.items()}
    got = {k: _rows(v, rows) for k, v in out.items()}
    del d, out
    _free()
    hf = (h["terminated"], h["truncated"], h["bootstrap_value"], h["trunc_bootstrap"])
    if name == "discounted_returns":
        ref = {"out": oracle.discounted_returns(h["r"], *hf, gamma=0.99)}
    elif name == "gae":
        a, r_ = oracle.gae(h["r"], h["v"], *hf, gamma=0.99, lam=0.95, with_returns=True)
        ref = {"out": a, "out1": r_}
    else:
        ref = {"out": oracle.retrace(h["r"], h["q"], h["exp_q"], h["pi"], h["mu"], *hf, gamma=0.99, lam=0.95)}
    for k in ref:
        err = parity_err(got[k], ref[k])
        assert err <= TOL, (name, k, err)


def test_time_major_past_2pow31_elements():
    import linear_recurrence_scan_reverse_amd as rl
    E, T = E_BIG, T_BIG
    _say("max sizes time-major td_lambda E=%d T=%d" % (E, T))
    d = _inputs((T, E), 91, ["r", "v", "trunc_bootstrap", "terminated", "truncated"])
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(92)
    bv = torch.randn(E, generator=g, device="cuda")
    out = rl.td_lambda(d["r"], d["v"], d["terminated"], d["truncated"], bv, d["trunc_bootstrap"], gamma=0.99,
                       lam=0.95, time_major=True)
    rows = _sample_rows(E, T)
    h = {k: _rows(v, rows, time_major=True) for k, v in d.items()}
    hb = _rows(bv, rows)
    got = _rows(out, rows, time_major=True)
    del d, out, bv
    _free()
    ref = oracle.td_lambda(h["r"], h["v"], h["terminated"], h["truncated"], hb, h["trunc_bootstrap"], gamma=0.99,
                           lam=0.95)
    assert parity_err(got, ref) <= TOL


def test_time_major_item_form_past_2pow31_elements():
    # the largest environment count of the LDS-staged item form (a multiple of
    # 64 below 2^23), with columns long enough to pass element 2^31
    import linear_recurrence_scan_reverse_amd as rl
    E, T = (1 << 23) - 64, 320
    _say("max sizes time-major item form td_lambda E=%d T=%d" % (E, T))
    d = _inputs((T, E), 93, ["r", "v", "trunc_bootstrap", "terminated", "truncated"])
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(94)
    bv = torch.randn(E, generator=g, device="cuda")
    out = rl.td_lambda(d["r"], d["v"], d["terminated"], d["truncated"], bv, d["trunc_bootstrap"], gamma=0.99,
                       lam=0.95, time_major=True)
    rows = _sample_rows(E, T)
    h = {k: _rows(v, rows, time_major=True) for k, v in d.items()}
    hb = _rows(bv, rows)
    got = _rows(out, rows, time_major=True)
    del d, out, bv
    _free()
    ref = oracle.td_lambda(h["r"], h["v"], h["terminated"], h["truncated"], hb, h["trunc_bootstrap"], gamma=0.99,
                           lam=0.95)
    assert parity_err(got, ref) <= TOL


def _episode_slices(done_row, n, backward, rng, span=4096):
    """n slices [a, b) of one row that contain whole episodes: backward, b - 1 is
    a terminated step; forward, a - 1 is a done step (or a = 0)."""
    idx = np.flatnonzero(done_row)
    out = []
    for j in rng.choice(len(idx) - 2, size=n, replace=False) + 1:
        if backward:
            b = int(idx[j]) + 1
            out.append((max(0, b - span), b))
        else:
            a = int(idx[j]) + 1
            out.append((a, min(len(done_row), a + span)))
    return out


def test_longest_rows_on_the_segmented_path():
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    E, T = 2, (1 << 30) - 1
    _say("max sizes segmented E=%d T=%d" % (E, T))
    d = _inputs((E, T), 93, ["r", "terminated"])
    g = torch.Generator(device="cuda")
    g.manual_seed(94)
    init = torch.randn(E, generator=g, device="cuda")
    dr = rl.discounted_returns(d["r"], d["terminated"], gamma=0.99)
    ps = rl.episodic_prefix_sum(d["r"], d["terminated"], None, init)
    rng = np.random.default_rng(95)
    for e in range(E):
        term = d["terminated"][e].cpu().numpy()
        # the row's last steps (a plain window end, bootstrap 0) and its first
        # steps (the carry-in) as well as sampled whole episodes
        last_cut = int(np.flatnonzero(term)[-1])
        first_cut = int(np.flatnonzero(term)[0])
        cases = [((last_cut + 1, T), "dr"), ((0, first_cut + 1), "ps")]
        cases += [(s, "dr") for s in _episode_slices(term, 4, True, rng)]
        cases += [(s, "ps") for s in _episode_slices(term, 4, False, rng)]
        for (a, b), kind in cases:
            r = d["r"][e, a:b].cpu().numpy()[None]
            tt = term[a:b][None]
            if kind == "dr":
                ref = oracle.discounted_returns(r, tt, gamma=0.99)
                got = dr[e, a:b].cpu().numpy()[None]
            else:
                i0 = init[e:e + 1].cpu().numpy() if a == 0 else None
                ref = oracle.episodic_prefix_sum(r, tt, None, i0)
                got = ps[e, a:b].cpu().numpy()[None]
            err = parity_err(got, ref)
            assert err <= TOL, (e, a, b, kind, err)
    del d, dr, ps, init
    _free()
