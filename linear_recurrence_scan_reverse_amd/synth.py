"""Seeded synthetic rollout inputs.

This module only draws random numbers; it holds none of the estimators'
arithmetic.  Both the GPU path's tests/benchmark and the CPU oracle's checks
take their inputs from here, so the two sides see identical bytes.

The rollout regime is the one the rl-triton pages benchmark (arxivlens.com
paper view, Abstract; gist.science summary, "Resultaten"): many parallel
environments, short rollouts, tensors shaped [num_envs, seq_len], with
terminated and truncated episode flags.  The pages name no dataset and print
no input distributions, so every distribution below is a stated choice.

Draw order is fixed so that a given (shape, seed) always produces the same
arrays: r, v, log_rhos, q, exp_q, pi, mu, bootstrap_value, trunc_bootstrap,
terminated, truncated.  Only the arrays a workload asks for are drawn.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ARRAY_ORDER = ("r", "v", "log_rhos", "q", "exp_q", "pi", "mu",
               "bootstrap_value", "trunc_bootstrap", "terminated", "truncated")


@dataclass(frozen=True)
class Workload:
    """One synthetic rollout workload: shape, distributions and parameters."""
    name: str
    estimators: tuple
    E: int
    T: int
    arrays: tuple
    p_term: float = 0.0
    p_trunc: float = 0.0
    logrho_std: float = 0.3
    prob_low: float = 0.05
    prob_high: float = 1.0
    gamma: float = 0.99
    lam: float = 0.95
    vtrace_lam: float = 1.0
    rho_bar: float = 1.0
    c_bar: float = 1.0
    seed: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)


ALL7 = ("discounted_returns", "td_lambda", "gae", "vtrace", "retrace",
        "eligibility_traces", "episodic_prefix_sum")

# The five workloads: sizes and distributions of the rl-triton regime.
WORKLOADS = {
    "gae_64x128": Workload(
        name="gae_64x128", estimators=("gae",), E=64, T=128,
        arrays=("r", "v", "bootstrap_value", "terminated"),
        p_term=0.01, p_trunc=0.0, gamma=0.99, lam=0.95,
        notes="GAE only; no truncation flags"),
    "dr_td_4096x64": Workload(
        name="dr_td_4096x64", estimators=("discounted_returns", "td_lambda"), E=4096, T=64,
        arrays=("r", "v", "bootstrap_value", "trunc_bootstrap", "terminated", "truncated"),
        p_term=0.01, p_trunc=0.005, gamma=0.99, lam=0.9,
        notes="bootstrap value supplied at truncations"),
    "vtrace_8192x128": Workload(
        name="vtrace_8192x128", estimators=("vtrace",), E=8192, T=128,
        arrays=("r", "v", "log_rhos", "bootstrap_value", "trunc_bootstrap",
                "terminated", "truncated"),
        p_term=0.005, p_trunc=0.005, gamma=0.99, lam=1.0, vtrace_lam=1.0,
        rho_bar=1.0, c_bar=1.0, notes="IMPALA lambda = 1"),
    "retrace_2048x1024": Workload(
        name="retrace_2048x1024", estimators=("retrace",), E=2048, T=1024,
        arrays=("r", "q", "exp_q", "pi", "mu", "bootstrap_value", "terminated"),
        p_term=0.002, p_trunc=0.0, gamma=0.99, lam=0.95,
        notes="long rollouts; no truncation flags"),
    "all7_16384x256": Workload(
        name="all7_16384x256", estimators=ALL7, E=16384, T=256,
        arrays=ARRAY_ORDER,
        p_term=0.004, p_trunc=0.004, gamma=0.99, lam=0.95, vtrace_lam=1.0,
        rho_bar=1.0, c_bar=1.0,
        notes="all seven estimators; rewards double as the trace/prefix signal"),
}


def draw(E: int, T: int, arrays=ARRAY_ORDER, *, seed: int = 0, p_term: float = 0.0,
         p_trunc: float = 0.0, logrho_std: float = 0.3, prob_low: float = 0.05,
         prob_high: float = 1.0) -> dict:
    """Draw the requested arrays in the fixed order with numpy's default_rng(seed).

    Returns a dict of numpy arrays: float32 [E, T] for r, v, log_rhos, q, exp_q,
    pi, mu, trunc_bootstrap; float32 [E] for bootstrap_value; uint8 [E, T]
    (0/1) for terminated and truncated.
    """
    wanted = set(arrays)
    unknown = wanted - set(ARRAY_ORDER)
    if unknown:
        raise ValueError("unknown arrays: %s" % sorted(unknown))
    rng = np.random.default_rng(seed)
    shape = (int(E), int(T))
    out = {}
    for name in ARRAY_ORDER:
        if name not in wanted:
            continue
        if name in ("r", "v", "q", "exp_q", "trunc_bootstrap"):
            out[name] = rng.standard_normal(shape, dtype=np.float32)
        elif name == "log_rhos":
            out[name] = (rng.standard_normal(shape, dtype=np.float32)
                         * np.float32(logrho_std)).astype(np.float32)
        elif name in ("pi", "mu"):
            out[name] = rng.uniform(prob_low, prob_high, size=shape).astype(np.float32)
        elif name == "bootstrap_value":
            out[name] = rng.standard_normal((shape[0],), dtype=np.float32)
        elif name == "terminated":
            out[name] = (rng.random(shape) < p_term).astype(np.uint8)
        elif name == "truncated":
            out[name] = (rng.random(shape) < p_trunc).astype(np.uint8)
    return out


def workload_inputs(w: Workload, *, E: int | None = None, T: int | None = None,
                    seed: int | None = None) -> dict:
    """Inputs for a named workload (optionally at another shape or seed)."""
    return draw(w.E if E is None else E, w.T if T is None else T, w.arrays,
                seed=w.seed if seed is None else seed, p_term=w.p_term, p_trunc=w.p_trunc,
                logrho_std=w.logrho_std, prob_low=w.prob_low, prob_high=w.prob_high)


def flag_patterns(T: int):
    """Every (terminated, truncated) pattern of length T: 4**T rows of uint8 flags.

    Row k encodes step t's pair as base-4 digit t of k: digit 0 = neither,
    1 = terminated, 2 = truncated, 3 = both.
    """
    n = 4 ** T
    k = np.arange(n, dtype=np.int64)
    digits = np.stack([(k // (4 ** t)) % 4 for t in range(T)], axis=1)
    term = ((digits & 1) != 0).astype(np.uint8)
    trunc = ((digits & 2) != 0).astype(np.uint8)
    return term, trunc


def draw_features(E: int, T: int, D: int, *, seed: int = 0, p_term: float = 0.0,
                  p_trunc: float = 0.0) -> dict:
    """Per-step feature vectors for the vector traces: x float32 [E, T, D] ~ N(0,1),
    init float32 [E, D] ~ N(0,1), terminated / truncated uint8 [E, T] ~ Bernoulli."""
    rng = np.random.default_rng(seed)
    return {
        "x": rng.standard_normal((int(E), int(T), int(D)), dtype=np.float32),
        "init": rng.standard_normal((int(E), int(D)), dtype=np.float32),
        "terminated": (rng.random((int(E), int(T))) < p_term).astype(np.uint8),
        "truncated": (rng.random((int(E), int(T))) < p_trunc).astype(np.uint8),
    }
