"""The bench's streaming-ceiling probe library (libstreamprobe.so, built beside
librlscan.so): it loads, exports its one entry point, and rejects arguments
outside its contract before any HIP call (so this runs without a GPU)."""
from __future__ import annotations

import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "linear_recurrence_scan_reverse_amd", "libstreamprobe.so")


@pytest.fixture(scope="module")
def fn():
    if not os.path.exists(PROBE):
        pytest.skip("libstreamprobe.so not built (python -m linear_recurrence_scan_reverse_amd.build)")
    f = ctypes.CDLL(PROBE).stream_probe
    P = ctypes.POINTER(ctypes.c_void_p)
    f.restype = ctypes.c_int
    f.argtypes = [P, ctypes.c_int, P, ctypes.c_int, P, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]
    return f


def _ptrs(*vals):
    return (ctypes.c_void_p * max(1, len(vals)))(*vals)


@pytest.mark.parametrize("nr,nf,nw,n", [(0, 0, 1, 16), (6, 0, 1, 16), (1, 3, 1, 16), (1, 0, 0, 16),
                                         (1, 0, 3, 16), (1, 0, 1, 0), (1, 0, 1, 6), (1, 0, 1, -4)])
def test_rejects_counts_and_sizes(fn, nr, nf, nw, n):
    a = _ptrs(*([16] * 5))
    f = _ptrs(4, 8)
    o = _ptrs(16, 32)
    assert fn(a, nr, f, nf, o, nw, n, None) == -1


def test_rejects_null_and_misaligned_pointers(fn):
    good_in, good_out = _ptrs(16), _ptrs(32)
    assert fn(None, 1, None, 0, good_out, 1, 16, None) == -1          # no input table
    assert fn(good_in, 1, None, 0, None, 1, 16, None) == -1           # no output table
    assert fn(good_in, 1, None, 1, good_out, 1, 16, None) == -1       # flags requested, no table
    assert fn(_ptrs(0), 1, None, 0, good_out, 1, 16, None) == -1      # NULL input
    assert fn(_ptrs(8), 1, None, 0, good_out, 1, 16, None) == -1      # input not 16-byte aligned
    assert fn(good_in, 1, _ptrs(2), 1, good_out, 1, 16, None) == -1  # flags not 4-byte aligned
    assert fn(good_in, 1, None, 0, _ptrs(4), 1, 16, None) == -1       # output not 16-byte aligned
