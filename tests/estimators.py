"""One place that maps each estimator to its GPU call and its oracle call.

Both sides receive the same numpy inputs (from linear_recurrence_scan_reverse_amd.synth)
and the same parameters; ``variant`` switches optional inputs off (NULL) so
that every code path of the ABI is exercised against the oracle.
"""
from __future__ import annotations

import numpy as np

import oracle

NAMES = ("discounted_returns", "td_lambda", "gae", "vtrace", "retrace",
         "eligibility_traces", "episodic_prefix_sum", "returns_and_td_lambda")

DEFAULT_PARAMS = dict(gamma=0.99, lam=0.95, vtrace_lam=1.0, rho_bar=1.0, c_bar=1.0)

# Parity metric: max_i |g_i - r_i| / max(1, |r_i|)  (relative where |r| >= 1,
# absolute below); the gate is 1e-5.
TOL = 1e-5


def parity_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref))))


def select(d, term=True, trunc=True, boot=True, tboot=True):
    """The optional inputs actually passed (None = NULL pointer)."""
    return dict(
        terminated=d.get("terminated") if term else None,
        truncated=d.get("truncated") if trunc else None,
        bootstrap_value=d.get("bootstrap_value") if boot else None,
        trunc_bootstrap=d.get("trunc_bootstrap") if tboot else None,
    )


def run_oracle(name, d, P=None, **variant):
    P = {**DEFAULT_PARAMS, **(P or {})}
    o = select(d, **variant)
    te, tr, bv, tb = o["terminated"], o["truncated"], o["bootstrap_value"], o["trunc_bootstrap"]
    g, l = P["gamma"], P["lam"]
    if name == "discounted_returns":
        return {"out": oracle.discounted_returns(d["r"], te, tr, bv, tb, gamma=g)}
    if name == "td_lambda":
        return {"out": oracle.td_lambda(d["r"], d["v"], te, tr, bv, tb, gamma=g, lam=l)}
    if name == "returns_and_td_lambda":
        return {"out": oracle.discounted_returns(d["r"], te, tr, bv, tb, gamma=g),
                "out1": oracle.td_lambda(d["r"], d["v"], te, tr, bv, tb, gamma=g, lam=l)}
    if name == "gae":
        adv, ret = oracle.gae(d["r"], d["v"], te, tr, bv, tb, gamma=g, lam=l, with_returns=True)
        return {"out": adv, "out1": ret}
    if name == "vtrace":
        vs, pg = oracle.vtrace(d["r"], d["v"], d["log_rhos"], te, tr, bv, tb, gamma=g,
                               lam=P["vtrace_lam"], rho_bar=P["rho_bar"], c_bar=P["c_bar"])
        return {"out": vs, "out1": pg}
    if name == "retrace":
        return {"out": oracle.retrace(d["r"], d["q"], d["exp_q"], d["pi"], d["mu"], te, tr, bv, tb,
                                      gamma=g, lam=l)}
    if name == "eligibility_traces":
        return {"out": oracle.eligibility_traces(d["r"], te, tr, bv, gamma=g, lam=l)}
    if name == "episodic_prefix_sum":
        return {"out": oracle.episodic_prefix_sum(d["r"], te, tr, bv)}
    raise KeyError(name)


def to_dev(d, device="cuda"):
    import torch
    return {k: (torch.from_numpy(np.ascontiguousarray(v)).to(device) if v is not None else None)
            for k, v in d.items()}


def run_gpu(name, dd, P=None, **variant):
    """dd: dict of device tensors (to_dev).  Returns a dict of device tensors."""
    import linear_recurrence_scan_reverse_amd as rl
    P = {**DEFAULT_PARAMS, **(P or {})}
    o = select(dd, **variant)
    te, tr, bv, tb = o["terminated"], o["truncated"], o["bootstrap_value"], o["trunc_bootstrap"]
    g, l = P["gamma"], P["lam"]
    if name == "discounted_returns":
        return {"out": rl.discounted_returns(dd["r"], te, tr, bv, tb, gamma=g)}
    if name == "td_lambda":
        return {"out": rl.td_lambda(dd["r"], dd["v"], te, tr, bv, tb, gamma=g, lam=l)}
    if name == "returns_and_td_lambda":
        ret, tdr = rl.returns_and_td_lambda(dd["r"], dd["v"], te, tr, bv, tb, gamma=g, lam=l)
        return {"out": ret, "out1": tdr}
    if name == "gae":
        adv, ret = rl.gae(dd["r"], dd["v"], te, tr, bv, tb, gamma=g, lam=l, with_returns=True)
        return {"out": adv, "out1": ret}
    if name == "vtrace":
        vs, pg = rl.vtrace(dd["r"], dd["v"], dd["log_rhos"], te, tr, bv, tb, gamma=g,
                           lam=P["vtrace_lam"], rho_bar=P["rho_bar"], c_bar=P["c_bar"])
        return {"out": vs, "out1": pg}
    if name == "retrace":
        return {"out": rl.retrace(dd["r"], dd["q"], dd["exp_q"], dd["pi"], dd["mu"], te, tr, bv, tb,
                                  gamma=g, lam=l)}
    if name == "eligibility_traces":
        return {"out": rl.eligibility_traces(dd["r"], te, tr, bv, gamma=g, lam=l)}
    if name == "episodic_prefix_sum":
        return {"out": rl.episodic_prefix_sum(dd["r"], te, tr, bv)}
    raise KeyError(name)


def compare(name, d, P=None, device="cuda", **variant):
    """Run both sides; return {output: (err, max|ref|)}."""
    import torch
    dd = to_dev(d, device)
    got = run_gpu(name, dd, P, **variant)
    torch.cuda.synchronize()
    ref = run_oracle(name, d, P, **variant)
    res = {}
    for k, r in ref.items():
        g = got[k].cpu().numpy()
        res[k] = (parity_err(g, r), float(np.max(np.abs(r))) if r.size else 0.0)
    return res
