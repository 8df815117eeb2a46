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


@pytest.mark.gpu
@pytest.mark.parametrize("nr,nf,nw", [(1, 2, 1), (2, 2, 1), (3, 2, 2), (5, 2, 1), (1, 0, 1), (4, 1, 2)])
def test_probe_moves_every_array(fn, nr, nf, nw):
    """The probe reads every input and flag array and writes every output: output k
    is the elementwise sum of the inputs plus k, plus 1 in lane x of a 4-element
    group whose flag bytes are not all zero."""
    import torch
    n = 4 * 1000
    g = torch.Generator(device="cpu").manual_seed(nr * 100 + nf * 10 + nw)
    ins = [torch.randn(n, generator=g).cuda() for _ in range(nr)]
    fls = [(torch.rand(n, generator=g) < 0.05).to(torch.uint8).cuda() for _ in range(nf)]
    outs = [torch.full((n,), float("nan"), device="cuda") for _ in range(nw)]
    rc = fn(_ptrs(*[t.data_ptr() for t in ins]), nr, _ptrs(*[t.data_ptr() for t in fls]), nf,
            _ptrs(*[t.data_ptr() for t in outs]), nw, n, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    ref = torch.stack([t.cpu() for t in ins]).sum(0).view(-1, 4)
    if nf:
        any_flag = torch.stack([t.cpu() for t in fls]).amax(0).view(-1, 4).amax(1) > 0
        ref[:, 0] += any_flag.float()
    for k, o in enumerate(outs):
        assert torch.allclose(o.cpu().view(-1, 4), ref + k, rtol=1e-6, atol=1e-5), "output %d" % k


@pytest.mark.gpu
@pytest.mark.parametrize("shape", range(6))
@pytest.mark.parametrize("nr,nf,nw", [(1, 2, 1), (5, 2, 1), (3, 2, 2)])
def test_every_probe_shape_moves_every_array(shape, nr, nf, nw):
    """Each shape of the bench's ceiling sweep, run through the timing entry point
    on one buffer set, writes what the single-shape probe writes (ragged n: the
    last block and tile are partial)."""
    import torch
    lib = ctypes.CDLL(PROBE)
    f = lib.stream_probe_time
    P = ctypes.POINTER(ctypes.c_void_p)
    f.restype = ctypes.c_int
    f.argtypes = [P, ctypes.c_int, P, ctypes.c_int, P, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
    assert lib.stream_probe_shapes() == 6
    n = 4 * 70001
    g = torch.Generator(device="cpu").manual_seed(shape * 1000 + nr * 100 + nf * 10 + nw)
    ins = [torch.randn(n, generator=g).cuda() for _ in range(nr)]
    fls = [(torch.rand(n, generator=g) < 0.05).to(torch.uint8).cuda() for _ in range(nf)]
    outs = [torch.full((n,), float("nan"), device="cuda") for _ in range(nw)]
    us = ctypes.c_float(0.0)
    rc = f(_ptrs(*[t.data_ptr() for t in ins]), nr, _ptrs(*[t.data_ptr() for t in fls]), nf,
           _ptrs(*[t.data_ptr() for t in outs]), nw, n, 1, shape, 3,
           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), ctypes.byref(us))
    assert rc == 0 and us.value > 0
    torch.cuda.synchronize()
    ref = torch.stack([t.cpu() for t in ins]).sum(0).view(-1, 4)
    any_flag = torch.stack([t.cpu() for t in fls]).amax(0).view(-1, 4).amax(1) > 0
    ref[:, 0] += any_flag.float()
    for k, o in enumerate(outs):
        assert torch.allclose(o.cpu().view(-1, 4), ref + k, rtol=1e-6, atol=1e-5), "shape %d output %d" % (shape, k)
