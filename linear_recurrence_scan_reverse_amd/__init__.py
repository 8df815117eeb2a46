"""RL credit-assignment estimators as one-pass affine scans on MI355X (gfx950).

Thin binding over the C ABI of ``librlscan.so`` (declared in include/rlscan.h).
Every function here only checks and marshals torch tensors (device, dtype,
contiguity, shape) and calls the matching ``rlscan_*`` entry point on the
current HIP stream; all arithmetic runs in the library's HIP kernels.  There is
no fallback: if the library is not built or cannot be loaded, every call raises.

Estimators (rl-triton, arxivlens.com paper view, Abstract): discounted returns,
TD(lambda) returns, GAE, V-trace, Retrace(lambda), eligibility traces and
episodic prefix sums, plus the generic recurrence ``linear_scan``.

Storage dtype and layout: the seven estimators take float32, bfloat16 or
float16 value tensors (all of one dtype, taken from the first value argument)
and return outputs of that dtype.  With ``time_major=True`` every per-step
tensor is [T, E] instead of [E, T] (per-env tensors stay [E]).  16-bit or
time-major calls go to the ``rlscan_*_ex`` entries.  The scan itself always
runs in float64 on the GPU.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "RlscanError", "lib", "library_path", "version",
    "discounted_returns", "td_lambda", "returns_and_td_lambda", "gae", "vtrace", "retrace",
    "eligibility_traces", "eligibility_traces_vec", "episodic_prefix_sum", "linear_scan",
    "linear_scan_segmented",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librlscan.so")
_lock = threading.Lock()
_lib = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_int = ctypes.c_int

# Argument types of every entry point, in include/rlscan.h order.
_SIGNATURES = {
    "rlscan_discounted_returns": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp],
    "rlscan_td_lambda": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _f32, _vp],
    "rlscan_returns_and_td_lambda": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _f32, _vp],
    "rlscan_gae": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _f32, _vp],
    "rlscan_vtrace": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _f32, _f32, _f32, _vp],
    "rlscan_retrace": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _f32, _vp],
    "rlscan_eligibility_traces": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _f32, _vp],
    "rlscan_episodic_prefix_sum": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp],
    "rlscan_linear_scan": [_vp, _vp, _vp, _vp, _i64, _i64, _int, _vp],
    "rlscan_linear_scan_segmented": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, _vp],
    "rlscan_eligibility_traces_vec": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _f32, _vp],
}
# The _ex entries take the storage format and the layout first, then the float32
# entry's arguments.
_EX = ("rlscan_discounted_returns", "rlscan_td_lambda", "rlscan_returns_and_td_lambda", "rlscan_gae",
       "rlscan_vtrace", "rlscan_retrace", "rlscan_eligibility_traces", "rlscan_episodic_prefix_sum")
for _n in _EX + ("rlscan_linear_scan_segmented", "rlscan_eligibility_traces_vec"):
    _SIGNATURES[_n + "_ex"] = [_int, _int] + _SIGNATURES[_n]
del _n

# rlscan_format codes by storage dtype name
_FORMATS = {"float32": 0, "bfloat16": 1, "float16": 2}


class RlscanError(RuntimeError):
    """A librlscan call returned a non-OK status."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, _status_string(status), status))


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded librlscan.so with argument types set (raises if not built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                "librlscan.so is not built (%s); build it with "
                "`python -m linear_recurrence_scan_reverse_amd.build`" % _LIB_PATH)
        handle = ctypes.CDLL(_LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        handle.rlscan_status_string.argtypes = [ctypes.c_int]
        handle.rlscan_status_string.restype = ctypes.c_char_p
        handle.rlscan_version.argtypes = []
        handle.rlscan_version.restype = ctypes.c_char_p
        _lib = handle
        return handle


def _status_string(status: int) -> str:
    return lib().rlscan_status_string(int(status)).decode()


def version() -> str:
    return lib().rlscan_version().decode()


# ----------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _rows(x, name):
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if x.dim() != 2:
        raise ValueError("%s must be [E, T], got shape %s" % (name, tuple(x.shape)))
    return x


def _check_val(x, name, shape, device, dtype=None):
    """A value tensor: ``dtype`` (float32 when None), shape, device, contiguous."""
    torch = _torch()
    if x is None:
        return None
    dtype = torch.float32 if dtype is None else dtype
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if x.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, str(dtype).replace("torch.", ""), x.dtype))
    if tuple(x.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(x.shape)))
    if x.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, x.device, device))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return x


_check_f32 = _check_val


def _storage(x, name):
    """The storage dtype of a primary value tensor (float32, bfloat16 or float16)."""
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    key = str(x.dtype).replace("torch.", "")
    if key not in _FORMATS:
        raise TypeError("%s must be float32, bfloat16 or float16, got %s" % (name, x.dtype))
    return x.dtype


def _entry(fname, dtype, time_major, *args):
    """Call the float32 row-major entry, or its _ex variant (16-bit storage or time-major)."""
    key = str(dtype).replace("torch.", "")
    if key == "float32" and not time_major:
        _call(fname, *args)
    else:
        _call(fname + "_ex", _FORMATS[key], 1 if time_major else 0, *args)


def _dims(shape, time_major):
    """(E, T) from the shape of a per-step tensor."""
    return (shape[1], shape[0]) if time_major else (shape[0], shape[1])


def _check_flags(x, name, shape, device):
    torch = _torch()
    if x is None:
        return None
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if x.dtype == torch.bool:
        x = x.view(torch.uint8)
    if x.dtype != torch.uint8:
        raise TypeError("%s must be uint8 or bool, got %s" % (name, x.dtype))
    if tuple(x.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(x.shape)))
    if x.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, x.device, device))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return x


def _ptr(x):
    return None if x is None else x.data_ptr()


def _stream(device, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _out(x, name, shape, device, dtype=None):
    torch = _torch()
    dtype = torch.float32 if dtype is None else dtype
    if x is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _check_val(x, name, shape, device, dtype)


def _call(fname, *args):
    st = getattr(lib(), fname)(*args)
    if st != 0:
        raise RlscanError(st, fname)


def _prep(primary, name):
    x = _rows(primary, name)
    if x.device.type != "cuda":
        raise ValueError("%s must be on a GPU device, got %s" % (name, x.device))
    return x.shape, x.device


# ----------------------------------------------------------------- estimators
def discounted_returns(rewards, terminated=None, truncated=None, bootstrap_value=None,
                       trunc_bootstrap=None, *, time_major=False, gamma=0.99, out=None, stream=None):
    """Discounted returns G_t = r_t + gamma * G_{t+1}, cut and bootstrapped at episode ends."""
    shape, dev = _prep(rewards, "rewards")
    E, T = _dims(shape, time_major)
    dt = _storage(rewards, "rewards")
    r = _check_val(rewards, "rewards", shape, dev, dt)
    te = _check_flags(terminated, "terminated", shape, dev)
    tr = _check_flags(truncated, "truncated", shape, dev)
    bv = _check_val(bootstrap_value, "bootstrap_value", (E,), dev, dt)
    tb = _check_val(trunc_bootstrap, "trunc_bootstrap", shape, dev, dt)
    out = _out(out, "out", shape, dev, dt)
    _entry("rlscan_discounted_returns", dt, time_major, _ptr(r), _ptr(te), _ptr(tr), _ptr(bv), _ptr(tb), _ptr(out),
           E, T, float(gamma), _stream(dev, stream))
    return out


def td_lambda(rewards, values, terminated=None, truncated=None, bootstrap_value=None,
              trunc_bootstrap=None, *, time_major=False, gamma=0.99, lam=0.95, out=None, stream=None):
    """TD(lambda) returns (recursive lambda-return)."""
    shape, dev = _prep(rewards, "rewards")
    E, T = _dims(shape, time_major)
    dt = _storage(rewards, "rewards")
    r = _check_val(rewards, "rewards", shape, dev, dt)
    v = _check_val(values, "values", shape, dev, dt)
    te = _check_flags(terminated, "terminated", shape, dev)
    tr = _check_flags(truncated, "truncated", shape, dev)
    bv = _check_val(bootstrap_value, "bootstrap_value", (E,), dev, dt)
    tb = _check_val(trunc_bootstrap, "trunc_bootstrap", shape, dev, dt)
    out = _out(out, "out", shape, dev, dt)
    _entry("rlscan_td_lambda", dt, time_major, _ptr(r), _ptr(v), _ptr(te), _ptr(tr), _ptr(bv), _ptr(tb), _ptr(out),
           E, T, float(gamma), float(lam), _stream(dev, stream))
    return out


def returns_and_td_lambda(rewards, values, terminated=None, truncated=None, bootstrap_value=None,
                          trunc_bootstrap=None, *, time_major=False, gamma=0.99, lam=0.95, returns=None,
                          td_returns=None, stream=None):
    """Discounted returns and TD(lambda) returns of one rollout in one pass.

    Returns (returns, td_returns), equal to ``discounted_returns`` and
    ``td_lambda`` with the same arguments."""
    shape, dev = _prep(rewards, "rewards")
    E, T = _dims(shape, time_major)
    dt = _storage(rewards, "rewards")
    r = _check_val(rewards, "rewards", shape, dev, dt)
    v = _check_val(values, "values", shape, dev, dt)
    te = _check_flags(terminated, "terminated", shape, dev)
    tr = _check_flags(truncated, "truncated", shape, dev)
    bv = _check_val(bootstrap_value, "bootstrap_value", (E,), dev, dt)
    tb = _check_val(trunc_bootstrap, "trunc_bootstrap", shape, dev, dt)
    returns = _out(returns, "returns", shape, dev, dt)
    td_returns = _out(td_returns, "td_returns", shape, dev, dt)
    _entry("rlscan_returns_and_td_lambda", dt, time_major, _ptr(r), _ptr(v), _ptr(te), _ptr(tr), _ptr(bv),
           _ptr(tb), _ptr(returns), _ptr(td_returns), E, T, float(gamma), float(lam), _stream(dev, stream))
    return returns, td_returns


def gae(rewards, values, terminated=None, truncated=None, bootstrap_value=None,
        trunc_bootstrap=None, *, time_major=False, gamma=0.99, lam=0.95, with_returns=False, advantages=None,
        returns=None, stream=None):
    """Generalized advantage estimates; with_returns=True also returns A + V."""
    shape, dev = _prep(rewards, "rewards")
    E, T = _dims(shape, time_major)
    dt = _storage(rewards, "rewards")
    r = _check_val(rewards, "rewards", shape, dev, dt)
    v = _check_val(values, "values", shape, dev, dt)
    te = _check_flags(terminated, "terminated", shape, dev)
    tr = _check_flags(truncated, "truncated", shape, dev)
    bv = _check_val(bootstrap_value, "bootstrap_value", (E,), dev, dt)
    tb = _check_val(trunc_bootstrap, "trunc_bootstrap", shape, dev, dt)
    adv = _out(advantages, "advantages", shape, dev, dt)
    ret = _out(returns, "returns", shape, dev, dt) if (with_returns or returns is not None) else None
    _entry("rlscan_gae", dt, time_major, _ptr(r), _ptr(v), _ptr(te), _ptr(tr), _ptr(bv), _ptr(tb), _ptr(adv), _ptr(ret),
           E, T, float(gamma), float(lam), _stream(dev, stream))
    return (adv, ret) if ret is not None else adv


def vtrace(rewards, values, log_rhos, terminated=None, truncated=None, bootstrap_value=None,
           trunc_bootstrap=None, *, time_major=False, gamma=0.99, lam=1.0, rho_bar=1.0, c_bar=1.0, with_pg=True,
           vs=None, pg_advantages=None, stream=None):
    """V-trace targets vs (and policy-gradient advantages when with_pg)."""
    shape, dev = _prep(rewards, "rewards")
    E, T = _dims(shape, time_major)
    dt = _storage(rewards, "rewards")
    r = _check_val(rewards, "rewards", shape, dev, dt)
    v = _check_val(values, "values", shape, dev, dt)
    lr = _check_val(log_rhos, "log_rhos", shape, dev, dt)
    te = _check_flags(terminated, "terminated", shape, dev)
    tr = _check_flags(truncated, "truncated", shape, dev)
    bv = _check_val(bootstrap_value, "bootstrap_value", (E,), dev, dt)
    tb = _check_val(trunc_bootstrap, "trunc_bootstrap", shape, dev, dt)
    vs = _out(vs, "vs", shape, dev, dt)
    pg = _out(pg_advantages, "pg_advantages", shape, dev, dt) if (with_pg or pg_advantages is not None) else None
    _entry("rlscan_vtrace", dt, time_major, _ptr(r), _ptr(v), _ptr(lr), _ptr(te), _ptr(tr), _ptr(bv), _ptr(tb),
           _ptr(vs), _ptr(pg), E, T, float(gamma), float(lam), float(rho_bar), float(c_bar),
           _stream(dev, stream))
    return (vs, pg) if pg is not None else vs


def retrace(rewards, q_values, expected_q, pi_prob, mu_prob, terminated=None, truncated=None,
            bootstrap_value=None, trunc_bootstrap=None, *, time_major=False, gamma=0.99, lam=0.95, out=None,
            stream=None):
    """Retrace(lambda) targets Q^ret."""
    shape, dev = _prep(rewards, "rewards")
    E, T = _dims(shape, time_major)
    dt = _storage(rewards, "rewards")
    r = _check_val(rewards, "rewards", shape, dev, dt)
    q = _check_val(q_values, "q_values", shape, dev, dt)
    eq = _check_val(expected_q, "expected_q", shape, dev, dt)
    pi = _check_val(pi_prob, "pi_prob", shape, dev, dt)
    mu = _check_val(mu_prob, "mu_prob", shape, dev, dt)
    te = _check_flags(terminated, "terminated", shape, dev)
    tr = _check_flags(truncated, "truncated", shape, dev)
    bv = _check_val(bootstrap_value, "bootstrap_value", (E,), dev, dt)
    tb = _check_val(trunc_bootstrap, "trunc_bootstrap", shape, dev, dt)
    out = _out(out, "out", shape, dev, dt)
    _entry("rlscan_retrace", dt, time_major, _ptr(r), _ptr(q), _ptr(eq), _ptr(pi), _ptr(mu), _ptr(te), _ptr(tr),
           _ptr(bv), _ptr(tb), _ptr(out), E, T, float(gamma), float(lam), _stream(dev, stream))
    return out


def eligibility_traces(x, terminated=None, truncated=None, init=None, *, time_major=False, gamma=0.99, lam=0.95,
                       out=None, stream=None):
    """Accumulating eligibility traces of x, forward in time, reset after each episode end."""
    shape, dev = _prep(x, "x")
    E, T = _dims(shape, time_major)
    dt = _storage(x, "x")
    xx = _check_val(x, "x", shape, dev, dt)
    te = _check_flags(terminated, "terminated", shape, dev)
    tr = _check_flags(truncated, "truncated", shape, dev)
    i0 = _check_val(init, "init", (E,), dev, dt)
    out = _out(out, "out", shape, dev, dt)
    _entry("rlscan_eligibility_traces", dt, time_major, _ptr(xx), _ptr(te), _ptr(tr), _ptr(i0), _ptr(out), E, T,
           float(gamma), float(lam), _stream(dev, stream))
    return out


def episodic_prefix_sum(x, terminated=None, truncated=None, init=None, *, time_major=False, out=None, stream=None):
    """Inclusive prefix sums of x within each episode, forward in time."""
    shape, dev = _prep(x, "x")
    E, T = _dims(shape, time_major)
    dt = _storage(x, "x")
    xx = _check_val(x, "x", shape, dev, dt)
    te = _check_flags(terminated, "terminated", shape, dev)
    tr = _check_flags(truncated, "truncated", shape, dev)
    i0 = _check_val(init, "init", (E,), dev, dt)
    out = _out(out, "out", shape, dev, dt)
    _entry("rlscan_episodic_prefix_sum", dt, time_major, _ptr(xx), _ptr(te), _ptr(tr), _ptr(i0), _ptr(out), E, T,
           _stream(dev, stream))
    return out


def linear_scan(a, b, carry=None, *, reverse=True, time_major=False, out=None, stream=None):
    """The generic recurrence x_t = a_t x_{t+1} + b_t (reverse) or x_t = a_t x_{t-1} + b_t."""
    return linear_scan_segmented(a, b, None, carry, reverse=reverse, time_major=time_major, out=out,
                                 stream=stream)


def linear_scan_segmented(a, b, done=None, carry=None, *, reverse=True, time_major=False, out=None,
                          stream=None):
    """The generic recurrence cut into episodes: a step flagged in ``done`` breaks
    the chain (backward: nothing enters it from t+1; forward: the next step
    starts afresh).  float32, bfloat16 or float16 values (the dtype of ``a``);
    ``time_major`` takes [T, E] arrays."""
    shape, dev = _prep(a, "a")
    E, T = _dims(shape, time_major)
    dt = _storage(a, "a")
    aa = _check_val(a, "a", shape, dev, dt)
    bb = _check_val(b, "b", shape, dev, dt)
    dn = _check_flags(done, "done", shape, dev)
    c0 = _check_val(carry, "carry", (E,), dev, dt)
    out = _out(out, "out", shape, dev, dt)
    args = (_ptr(aa), _ptr(bb), _ptr(dn), _ptr(c0), _ptr(out), E, T, 1 if reverse else 0, _stream(dev, stream))
    if str(dt) == "torch.float32" and not time_major:
        if dn is None:
            _call("rlscan_linear_scan", args[0], args[1], args[3], args[4], *args[5:])
        else:
            _call("rlscan_linear_scan_segmented", *args)
    else:
        _call("rlscan_linear_scan_segmented_ex", _FORMATS[str(dt).replace("torch.", "")],
              1 if time_major else 0, *args)
    return out


def eligibility_traces_vec(x, terminated=None, truncated=None, init=None, *, gamma=0.99, lam=0.95,
                           time_major=False, out=None, stream=None):
    """Eligibility traces of feature vectors: x [E, T, D] (time_major: [T, E, D]),
    flags [E, T] ([T, E]), init [E, D]; every column follows the scalar trace
    with the row's flags.  float32, bfloat16 or float16 (the dtype of x)."""
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x must be a [E, T, D] tensor")
    if x.device.type != "cuda":
        raise ValueError("x must be on a GPU device, got %s" % x.device)
    if time_major:
        T, E, D = x.shape
    else:
        E, T, D = x.shape
    dev = x.device
    dt = _storage(x, "x")
    fshape = (T, E) if time_major else (E, T)
    xx = _check_val(x, "x", tuple(x.shape), dev, dt)
    te = _check_flags(terminated, "terminated", fshape, dev)
    tr = _check_flags(truncated, "truncated", fshape, dev)
    it = _check_val(init, "init", (E, D), dev, dt)
    out = _out(out, "out", tuple(x.shape), dev, dt)
    args = (_ptr(xx), _ptr(te), _ptr(tr), _ptr(it), _ptr(out), E, T, D, float(gamma), float(lam),
            _stream(dev, stream))
    _entry("rlscan_eligibility_traces_vec", dt, time_major, *args)
    return out
