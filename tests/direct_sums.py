"""Brute-force direct sums for the seven estimators (tiny inputs, pure Python).

These are the closed, non-recursive forms of each estimator -- finite sums of
discounted, trace-weighted terms up to the end of the episode segment -- so
they pin the oracle's backward/forward recursions with a formulation that
shares no steps with them.  O(T^2) or O(T^3) per row: tiny inputs only.

Definitions (standard published forms; the rl-triton pages name the
estimators but print no formulas):
  discounted   G_t = sum_{k<n} g^k r_{t+k} + g^n B
  lambda-ret   G^l_t = (1-l) sum_{m=1}^{n-1} l^{m-1} G^(m)_t + l^{n-1} G_t   (Sutton & Barto)
  GAE          A_t = sum_{k<n} (g l)^k delta_{t+k}                               (Schulman et al.)
  V-trace      vs_t = V_t + sum_{k<n} g^k (prod_{i=t}^{t+k-1} c_i) delta_{t+k}   (Espeholt et al.)
  Retrace      Qret_t = Q_t + sum_{k<n} g^k (prod_{i=t+1}^{t+k} c_i) delta_{t+k} (Munos et al.)
  trace        e_t = sum_{k=s}^{t} d^{t-k} x_k + [s=0] d^{t+1} init
  prefix sum   S_t = sum_{k=s}^{t} x_k + [s=0] init
with n the number of steps from t through the first step that is not a plain
continuation (terminated, truncated, or the window end), B that step's
successor value (0 / truncation bootstrap / row bootstrap), and s the first
step of t's episode for the forward estimators.
"""
from __future__ import annotations

import math

import numpy as np

CONT, TERM, TRUNC, END = 0, 1, 2, 3


def f32(x):
    """Parameters reach the kernels as float32; use the same rounded value."""
    return float(np.float32(x))


def _row(a, e):
    return None if a is None else [float(v) for v in np.asarray(a)[e]]


def _kinds(term, trunc, T):
    out = []
    for t in range(T):
        if term is not None and term[t]:
            out.append(TERM)
        elif trunc is not None and trunc[t]:
            out.append(TRUNC)
        elif t == T - 1:
            out.append(END)
        else:
            out.append(CONT)
    return out


def _seg_end(kinds, t):
    j = t
    while kinds[j] == CONT:
        j += 1
    return j


def _boot(kind, j, bv, tb):
    if kind == TERM:
        return 0.0
    if kind == TRUNC:
        return tb[j] if tb is not None else 0.0
    return bv if bv is not None else 0.0


def _successor(kinds, s, nextval, bv, tb):
    return nextval[s + 1] if kinds[s] == CONT else _boot(kinds[s], s, bv, tb)


def _per_row(fn, E, *arrays):
    return [fn(e, *[_row(a, e) for a in arrays]) for e in range(E)]


def _rowval(a, e):
    return None if a is None else float(np.asarray(a).reshape(-1)[e])


def discounted_returns(r, term=None, trunc=None, bv=None, tb=None, gamma=0.99):
    g = f32(gamma)
    E, T = np.asarray(r).shape
    out = np.zeros((E, T))
    for e in range(E):
        rr, te, tr, tbr = _row(r, e), _row(term, e), _row(trunc, e), _row(tb, e)
        b = _rowval(bv, e)
        kinds = _kinds(te, tr, T)
        for t in range(T):
            j = _seg_end(kinds, t)
            n = j - t + 1
            out[e, t] = sum(g ** k * rr[t + k] for k in range(n)) + g ** n * _boot(kinds[j], j, b, tbr)
    return out


def td_lambda(r, v, term=None, trunc=None, bv=None, tb=None, gamma=0.99, lam=0.95):
    g, l = f32(gamma), f32(lam)
    E, T = np.asarray(r).shape
    out = np.zeros((E, T))
    for e in range(E):
        rr, vv, te, tr, tbr = _row(r, e), _row(v, e), _row(term, e), _row(trunc, e), _row(tb, e)
        b = _rowval(bv, e)
        kinds = _kinds(te, tr, T)
        for t in range(T):
            j = _seg_end(kinds, t)
            n = j - t + 1
            full = sum(g ** k * rr[t + k] for k in range(n)) + g ** n * _boot(kinds[j], j, b, tbr)
            acc = 0.0
            for m in range(1, n):
                nstep = sum(g ** k * rr[t + k] for k in range(m)) + g ** m * vv[t + m]
                acc += l ** (m - 1) * nstep
            out[e, t] = (1.0 - l) * acc + l ** (n - 1) * full
    return out


def gae(r, v, term=None, trunc=None, bv=None, tb=None, gamma=0.99, lam=0.95):
    g, l = f32(gamma), f32(lam)
    E, T = np.asarray(r).shape
    out = np.zeros((E, T))
    for e in range(E):
        rr, vv, te, tr, tbr = _row(r, e), _row(v, e), _row(term, e), _row(trunc, e), _row(tb, e)
        b = _rowval(bv, e)
        kinds = _kinds(te, tr, T)
        delta = [rr[s] + g * _successor(kinds, s, vv, b, tbr) - vv[s] for s in range(T)]
        for t in range(T):
            j = _seg_end(kinds, t)
            out[e, t] = sum((g * l) ** k * delta[t + k] for k in range(j - t + 1))
    return out


def vtrace(r, v, log_rhos, term=None, trunc=None, bv=None, tb=None, gamma=0.99, lam=1.0,
           rho_bar=1.0, c_bar=1.0):
    g, l, rb, cb = f32(gamma), f32(lam), f32(rho_bar), f32(c_bar)
    E, T = np.asarray(r).shape
    vs = np.zeros((E, T))
    pg = np.zeros((E, T))
    for e in range(E):
        rr, vv, lr = _row(r, e), _row(v, e), _row(log_rhos, e)
        te, tr, tbr = _row(term, e), _row(trunc, e), _row(tb, e)
        b = _rowval(bv, e)
        kinds = _kinds(te, tr, T)
        ratio = [math.exp(x) for x in lr]
        rho = [min(rb, x) for x in ratio]
        c = [l * min(cb, x) for x in ratio]
        delta = [rho[s] * (rr[s] + g * _successor(kinds, s, vv, b, tbr) - vv[s]) for s in range(T)]
        for t in range(T):
            j = _seg_end(kinds, t)
            acc = 0.0
            for k in range(j - t + 1):
                acc += g ** k * math.prod(c[t:t + k]) * delta[t + k]
            vs[e, t] = vv[t] + acc
        for t in range(T):
            succ = vs[e, t + 1] if kinds[t] == CONT else _boot(kinds[t], t, b, tbr)
            pg[e, t] = rho[t] * (rr[t] + g * succ - vv[t])
    return vs, pg


def retrace(r, q, exp_q, pi, mu, term=None, trunc=None, bv=None, tb=None, gamma=0.99, lam=0.95):
    g, l = f32(gamma), f32(lam)
    E, T = np.asarray(r).shape
    out = np.zeros((E, T))
    for e in range(E):
        rr, qq, eq, pp, mm = _row(r, e), _row(q, e), _row(exp_q, e), _row(pi, e), _row(mu, e)
        te, tr, tbr = _row(term, e), _row(trunc, e), _row(tb, e)
        b = _rowval(bv, e)
        kinds = _kinds(te, tr, T)
        c = [l * min(1.0, pp[i] / mm[i]) for i in range(T)]
        delta = [rr[s] + g * _successor(kinds, s, eq, b, tbr) - qq[s] for s in range(T)]
        for t in range(T):
            j = _seg_end(kinds, t)
            acc = 0.0
            for k in range(j - t + 1):
                acc += g ** k * math.prod(c[t + 1:t + k + 1]) * delta[t + k]
            out[e, t] = qq[t] + acc
    return out


def _episode_start(done, t):
    s = 0
    for j in range(t):
        if done[j]:
            s = j + 1
    return s


def _dones(te, tr, T):
    return [bool((te is not None and te[t]) or (tr is not None and tr[t])) for t in range(T)]


def eligibility_traces(x, term=None, trunc=None, init=None, gamma=0.99, lam=0.95):
    d = f32(gamma) * f32(lam)
    E, T = np.asarray(x).shape
    out = np.zeros((E, T))
    for e in range(E):
        xx, te, tr = _row(x, e), _row(term, e), _row(trunc, e)
        i0 = _rowval(init, e) or 0.0
        done = _dones(te, tr, T)
        for t in range(T):
            s = _episode_start(done, t)
            acc = sum(d ** (t - k) * xx[k] for k in range(s, t + 1))
            if s == 0:
                acc += d ** (t + 1) * i0
            out[e, t] = acc
    return out


def episodic_prefix_sum(x, term=None, trunc=None, init=None):
    E, T = np.asarray(x).shape
    out = np.zeros((E, T))
    for e in range(E):
        xx, te, tr = _row(x, e), _row(term, e), _row(trunc, e)
        i0 = _rowval(init, e) or 0.0
        done = _dones(te, tr, T)
        for t in range(T):
            s = _episode_start(done, t)
            out[e, t] = sum(xx[s:t + 1]) + (i0 if s == 0 else 0.0)
    return out


def linear_scan(a, b, carry=None, reverse=True):
    E, T = np.asarray(a).shape
    out = np.zeros((E, T))
    for e in range(E):
        aa, bb = _row(a, e), _row(b, e)
        c0 = _rowval(carry, e) or 0.0
        for t in range(T):
            if reverse:
                acc = sum(math.prod(aa[t:j]) * bb[j] for j in range(t, T))
                acc += math.prod(aa[t:T]) * c0
            else:
                acc = sum(math.prod(aa[j + 1:t + 1]) * bb[j] for j in range(0, t + 1))
                acc += math.prod(aa[0:t + 1]) * c0
            out[e, t] = acc
    return out


def linear_scan_segmented(a, b, done=None, carry=None, reverse=True):
    """Episode-cut generic recurrence as a direct sum: backward, x_t sums b_j
    weighted by prod a_t..a_{j-1} for j from t through the first flagged step
    at or after t (the carry enters only if no step from t on is flagged);
    forward, x_t sums b_j weighted by prod a_{j+1}..a_t for j from the first
    step of t's episode (the step after the last flagged one before t) through
    t, plus the carry through a_0..a_t when that episode starts at 0."""
    E, T = np.asarray(a).shape
    out = np.zeros((E, T))
    for e in range(E):
        aa, bb = _row(a, e), _row(b, e)
        dd = [bool(x) for x in _row(done, e)] if done is not None else [False] * T
        c0 = _rowval(carry, e) or 0.0
        for t in range(T):
            if reverse:
                end = next((j for j in range(t, T) if dd[j]), None)
                last = T - 1 if end is None else end
                acc = sum(math.prod(aa[t:j]) * bb[j] for j in range(t, last + 1))
                if end is None:
                    acc += math.prod(aa[t:T]) * c0
            else:
                s0 = _episode_start(dd, t)
                acc = sum(math.prod(aa[j + 1:t + 1]) * bb[j] for j in range(s0, t + 1))
                if s0 == 0:
                    acc += math.prod(aa[0:t + 1]) * c0
            out[e, t] = acc
    return out
