"""fp64 CPU oracle for the RL credit-assignment estimators (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check in the package entry
file and the CPU-baseline leg of the benchmark may import this module; the
product path (the HIP library and its binding) never does, and shares no code
with it.  The arithmetic lives in ``rlscan_oracle.c`` (plain sequential C in
IEEE double); this module only builds it with gcc and marshals numpy arrays.

Every function takes numpy arrays shaped [E, T] (float32 inputs, uint8 flags,
[E] float32 per-row values) and returns float64 arrays of the same shape.  The
scalar parameters are rounded to float32 first, exactly as the GPU ABI receives
them, and upcast inside the C code.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rlscan_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64
_f32 = ctypes.c_float


def build(force: bool = True) -> str:
    """Compile rlscan_oracle.c into liboracle.so with gcc (-O2, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(lib):
    sig = {
        "oracle_discounted_returns": [_f32p, _u8p, _u8p, _f32p, _f32p, _f64p, _i64, _i64, _f32],
        "oracle_td_lambda": [_f32p, _f32p, _u8p, _u8p, _f32p, _f32p, _f64p, _i64, _i64, _f32, _f32],
        "oracle_gae": [_f32p, _f32p, _u8p, _u8p, _f32p, _f32p, _f64p, _f64p, _i64, _i64, _f32, _f32],
        "oracle_vtrace": [_f32p, _f32p, _f32p, _u8p, _u8p, _f32p, _f32p, _f64p, _f64p, _i64, _i64,
                          _f32, _f32, _f32, _f32],
        "oracle_retrace": [_f32p, _f32p, _f32p, _f32p, _f32p, _u8p, _u8p, _f32p, _f32p, _f64p,
                           _i64, _i64, _f32, _f32],
        "oracle_eligibility_traces": [_f32p, _u8p, _u8p, _f32p, _f64p, _i64, _i64, _f32, _f32],
        "oracle_episodic_prefix_sum": [_f32p, _u8p, _u8p, _f32p, _f64p, _i64, _i64],
        "oracle_linear_scan": [_f32p, _f32p, _f32p, _f64p, _i64, _i64, ctypes.c_int],
        "oracle_linear_scan_segmented": [_f32p, _f32p, _u8p, _f32p, _f64p, _i64, _i64, ctypes.c_int],
        "oracle_eligibility_traces_vec": [_f32p, _u8p, _u8p, _f32p, _f64p, _i64, _i64, _i64, _f32, _f32],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = None
    return lib


@contextlib.contextmanager
def use_library(path):
    """Temporarily route every wrapper to another build of the oracle source.

    Used only by the mutation tests, which compile deliberately wrong copies of
    rlscan_oracle.c and check that the pins reject them.
    """
    global _lib
    with _lock:
        saved = _lib
        _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        with _lock:
            _lib = saved


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
        return _lib


# ----------------------------------------------------------------- marshalling
def _shape(x):
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("expected a [E, T] array, got shape %r" % (x.shape,))
    return x.shape


def _f32_in(x, shape):
    if x is None:
        return None, None
    a = np.ascontiguousarray(x, dtype=np.float32)
    if a.shape != shape:
        raise ValueError("shape %r != %r" % (a.shape, shape))
    return a, a.ctypes.data_as(_f32p)


def _row_in(x, E):
    if x is None:
        return None, None
    a = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    if a.shape != (E,):
        raise ValueError("per-row array must have shape (%d,), got %r" % (E, a.shape))
    return a, a.ctypes.data_as(_f32p)


def _u8_in(x, shape):
    if x is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(x) != 0, dtype=np.uint8)
    if a.shape != shape:
        raise ValueError("shape %r != %r" % (a.shape, shape))
    return a, a.ctypes.data_as(_u8p)


def _out(shape):
    a = np.empty(shape, dtype=np.float64)
    return a, a.ctypes.data_as(_f64p)


def _p(x):
    return float(np.float32(x))


# ----------------------------------------------------------------- estimators
def discounted_returns(rewards, terminated=None, truncated=None, bootstrap_value=None,
                       trunc_bootstrap=None, gamma=0.99):
    shape = _shape(rewards)
    E, T = shape
    keep = [_f32_in(rewards, shape), _u8_in(terminated, shape), _u8_in(truncated, shape),
            _row_in(bootstrap_value, E), _f32_in(trunc_bootstrap, shape)]
    out, po = _out(shape)
    _load().oracle_discounted_returns(*(k[1] for k in keep), po, E, T, _p(gamma))
    return out


def td_lambda(rewards, values, terminated=None, truncated=None, bootstrap_value=None,
              trunc_bootstrap=None, gamma=0.99, lam=0.95):
    shape = _shape(rewards)
    E, T = shape
    keep = [_f32_in(rewards, shape), _f32_in(values, shape), _u8_in(terminated, shape),
            _u8_in(truncated, shape), _row_in(bootstrap_value, E), _f32_in(trunc_bootstrap, shape)]
    out, po = _out(shape)
    _load().oracle_td_lambda(*(k[1] for k in keep), po, E, T, _p(gamma), _p(lam))
    return out


def gae(rewards, values, terminated=None, truncated=None, bootstrap_value=None,
        trunc_bootstrap=None, gamma=0.99, lam=0.95, with_returns=False):
    shape = _shape(rewards)
    E, T = shape
    keep = [_f32_in(rewards, shape), _f32_in(values, shape), _u8_in(terminated, shape),
            _u8_in(truncated, shape), _row_in(bootstrap_value, E), _f32_in(trunc_bootstrap, shape)]
    adv, pa = _out(shape)
    ret, pr = _out(shape) if with_returns else (None, None)
    _load().oracle_gae(*(k[1] for k in keep), pa, pr, E, T, _p(gamma), _p(lam))
    return (adv, ret) if with_returns else adv


def vtrace(rewards, values, log_rhos, terminated=None, truncated=None, bootstrap_value=None,
           trunc_bootstrap=None, gamma=0.99, lam=1.0, rho_bar=1.0, c_bar=1.0, with_pg=True):
    shape = _shape(rewards)
    E, T = shape
    keep = [_f32_in(rewards, shape), _f32_in(values, shape), _f32_in(log_rhos, shape),
            _u8_in(terminated, shape), _u8_in(truncated, shape), _row_in(bootstrap_value, E),
            _f32_in(trunc_bootstrap, shape)]
    vs, pv = _out(shape)
    pg, pp = _out(shape) if with_pg else (None, None)
    _load().oracle_vtrace(*(k[1] for k in keep), pv, pp, E, T, _p(gamma), _p(lam),
                          _p(rho_bar), _p(c_bar))
    return (vs, pg) if with_pg else vs


def retrace(rewards, q_values, expected_q, pi_prob, mu_prob, terminated=None, truncated=None,
            bootstrap_value=None, trunc_bootstrap=None, gamma=0.99, lam=0.95):
    shape = _shape(rewards)
    E, T = shape
    keep = [_f32_in(rewards, shape), _f32_in(q_values, shape), _f32_in(expected_q, shape),
            _f32_in(pi_prob, shape), _f32_in(mu_prob, shape), _u8_in(terminated, shape),
            _u8_in(truncated, shape), _row_in(bootstrap_value, E), _f32_in(trunc_bootstrap, shape)]
    out, po = _out(shape)
    _load().oracle_retrace(*(k[1] for k in keep), po, E, T, _p(gamma), _p(lam))
    return out


def eligibility_traces(x, terminated=None, truncated=None, init=None, gamma=0.99, lam=0.95):
    shape = _shape(x)
    E, T = shape
    keep = [_f32_in(x, shape), _u8_in(terminated, shape), _u8_in(truncated, shape),
            _row_in(init, E)]
    out, po = _out(shape)
    _load().oracle_eligibility_traces(*(k[1] for k in keep), po, E, T, _p(gamma), _p(lam))
    return out


def episodic_prefix_sum(x, terminated=None, truncated=None, init=None):
    shape = _shape(x)
    E, T = shape
    keep = [_f32_in(x, shape), _u8_in(terminated, shape), _u8_in(truncated, shape),
            _row_in(init, E)]
    out, po = _out(shape)
    _load().oracle_episodic_prefix_sum(*(k[1] for k in keep), po, E, T)
    return out


def linear_scan(a, b, carry=None, reverse=True):
    shape = _shape(a)
    E, T = shape
    keep = [_f32_in(a, shape), _f32_in(b, shape), _row_in(carry, E)]
    out, po = _out(shape)
    _load().oracle_linear_scan(*(k[1] for k in keep), po, E, T, 1 if reverse else 0)
    return out


def linear_scan_segmented(a, b, done=None, carry=None, reverse=True):
    """The generic recurrence with episode cuts at flagged steps."""
    shape = _shape(a)
    E, T = shape
    keep = [_f32_in(a, shape), _f32_in(b, shape), _u8_in(done, shape), _row_in(carry, E)]
    out, po = _out(shape)
    _load().oracle_linear_scan_segmented(*(k[1] for k in keep), po, E, T, 1 if reverse else 0)
    return out


def eligibility_traces_vec(x, terminated=None, truncated=None, init=None, gamma=0.99, lam=0.95):
    """Eligibility traces of feature vectors: x [E, T, D], flags [E, T], init [E, D]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 3:
        raise ValueError("x must be [E, T, D]")
    E, T, D = x.shape
    te = _u8_in(terminated, (E, T))
    tr = _u8_in(truncated, (E, T))
    it = (None, None) if init is None else _f32_in(init, (E, D))
    out = np.empty((E, T, D), dtype=np.float64)
    _load().oracle_eligibility_traces_vec(x.ctypes.data_as(_f32p), te[1], tr[1], it[1],
                                          out.ctypes.data_as(_f64p), E, T, D,
                                          float(np.float32(gamma)), float(np.float32(lam)))
    return out


ESTIMATORS = ("discounted_returns", "td_lambda", "gae", "vtrace", "retrace",
              "eligibility_traces", "episodic_prefix_sum")
