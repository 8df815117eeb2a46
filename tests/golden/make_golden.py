"""Write tests/golden/oracle_small.json from the fp64 oracle (calls only oracle/).

The rl-triton pages print no worked numeric example, so there is no published
fixture to store.  This file instead freezes the oracle's own outputs on one
tiny seeded rollout (3 envs x 9 steps, flags at rate 0.2) so that any later
change to the oracle's arithmetic shows up as a diff of this fixture; such a
change must name, in its commit message, the passage or reading behind it.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from linear_recurrence_scan_reverse_amd import synth  # noqa: E402

E, T, SEED, P = 3, 9, 1234, 0.2
PARAMS = dict(gamma=0.99, lam=0.95, vtrace_lam=1.0, rho_bar=1.0, c_bar=1.0)


def compute(d):
    te, tr, bv, tb = d["terminated"], d["truncated"], d["bootstrap_value"], d["trunc_bootstrap"]
    g, l = PARAMS["gamma"], PARAMS["lam"]
    out = {}
    out["discounted_returns"] = oracle.discounted_returns(d["r"], te, tr, bv, tb, gamma=g)
    out["td_lambda"] = oracle.td_lambda(d["r"], d["v"], te, tr, bv, tb, gamma=g, lam=l)
    adv, ret = oracle.gae(d["r"], d["v"], te, tr, bv, tb, gamma=g, lam=l, with_returns=True)
    out["gae_advantages"], out["gae_returns"] = adv, ret
    vs, pg = oracle.vtrace(d["r"], d["v"], d["log_rhos"], te, tr, bv, tb, gamma=g,
                           lam=PARAMS["vtrace_lam"], rho_bar=PARAMS["rho_bar"], c_bar=PARAMS["c_bar"])
    out["vtrace_vs"], out["vtrace_pg"] = vs, pg
    out["retrace"] = oracle.retrace(d["r"], d["q"], d["exp_q"], d["pi"], d["mu"], te, tr, bv, tb,
                                    gamma=g, lam=l)
    out["eligibility_traces"] = oracle.eligibility_traces(d["r"], te, tr, bv, gamma=g, lam=l)
    out["episodic_prefix_sum"] = oracle.episodic_prefix_sum(d["r"], te, tr, bv)
    # the generic recurrence with cuts at the terminated steps: a = the
    # probabilities pi (in (0.05, 1)), b = rewards, carry = bootstrap_value
    for rev in (True, False):
        out["linear_scan_segmented_%s" % ("reverse" if rev else "forward")] = oracle.linear_scan_segmented(
            d["pi"], d["r"], te, bv, reverse=rev)
    # vector traces: features v (column 0), q (column 1), exp_q (column 2)
    import numpy as np
    x = np.ascontiguousarray(np.stack([d["v"], d["q"], d["exp_q"]], axis=-1))
    init = np.ascontiguousarray(np.stack([bv, bv, bv], axis=-1))
    tv = oracle.eligibility_traces_vec(x, te, tr, init, gamma=g, lam=l)
    for c in range(3):
        out["eligibility_traces_vec_col%d" % c] = np.ascontiguousarray(tv[:, :, c])
    return out


def inputs():
    return synth.draw(E, T, seed=SEED, p_term=P, p_trunc=P)


def main():
    d = inputs()
    out = compute(d)
    doc = {
        "about": "fp64 oracle outputs on synth.draw(3, 9, seed=1234, p_term=p_trunc=0.2); "
                 "written by tests/golden/make_golden.py",
        "shape": [E, T], "seed": SEED, "p": P, "params": PARAMS,
        "outputs": {k: [[float(x) for x in row] for row in v] for k, v in out.items()},
    }
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
