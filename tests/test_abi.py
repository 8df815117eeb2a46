"""C-ABI surface of librlscan (CPU only: no kernel is ever launched here).

* the library loads and exports every function include/rlscan.h declares;
* host-side validation returns the documented status before any HIP call
  (every call below fails validation, so no device is needed);
* the Python binding fails loudly when the library is missing.
"""
from __future__ import annotations

import math
import os
import re

import pytest

import linear_recurrence_scan_reverse_amd as rl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rlscan.h")

OK, ERR_NULL, ERR_SHAPE, ERR_PARAM, ERR_HIP, ERR_ALIGN, ERR_ALIAS = range(7)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rlscan_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rl.library_path()):
        from linear_recurrence_scan_reverse_amd import build
        build.build(verbose=False)
    return rl.lib()


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for n in ["rlscan_discounted_returns", "rlscan_td_lambda", "rlscan_returns_and_td_lambda",
              "rlscan_gae", "rlscan_vtrace",
              "rlscan_retrace", "rlscan_eligibility_traces", "rlscan_episodic_prefix_sum",
              "rlscan_linear_scan", "rlscan_linear_scan_segmented", "rlscan_eligibility_traces_vec",
              "rlscan_discounted_returns_ex", "rlscan_td_lambda_ex", "rlscan_returns_and_td_lambda_ex", "rlscan_gae_ex",
              "rlscan_vtrace_ex", "rlscan_retrace_ex", "rlscan_eligibility_traces_ex",
              "rlscan_episodic_prefix_sum_ex", "rlscan_linear_scan_segmented_ex", "rlscan_eligibility_traces_vec_ex",
              "rlscan_status_string",
              "rlscan_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), "librlscan.so does not export %s" % name


def test_version_and_status_strings(lib):
    assert "gfx950" in rl.version()
    for s in range(7):
        assert lib.rlscan_status_string(s)
    assert lib.rlscan_status_string(99) == b"unknown status"


# Fake, never-dereferenced device addresses (validation fails before any HIP call).
A = 0x7F0000000000
B = 0x7F0010000000
C = 0x7F0020000000
D = 0x7F0030000000
F = 0x7F0040000000
G = 0x7F0050000000
S = None  # default stream


def test_shape_errors(lib):
    assert lib.rlscan_gae(A, B, None, None, None, None, C, None, -1, 4, 0.99, 0.95, S) == ERR_SHAPE
    assert lib.rlscan_gae(A, B, None, None, None, None, C, None, 4, -1, 0.99, 0.95, S) == ERR_SHAPE
    assert lib.rlscan_gae(A, B, None, None, None, None, C, None, 2 ** 40, 2 ** 40, 0.99, 0.95, S) == ERR_SHAPE
    assert lib.rlscan_linear_scan(A, B, None, C, -3, 1, 1, S) == ERR_SHAPE
    # rows longer than 2^30 - 1 steps are rejected before any launch
    assert lib.rlscan_episodic_prefix_sum(A, None, None, None, C, 1, 2 ** 30, S) == ERR_SHAPE
    assert lib.rlscan_linear_scan(A, B, None, C, 1, 2 ** 30, 0, S) == ERR_SHAPE


@pytest.mark.parametrize("g,l", [(1.5, 0.9), (-0.1, 0.9), (0.9, 1.01), (math.nan, 0.5), (0.5, math.inf)])
def test_parameter_errors(lib, g, l):
    assert lib.rlscan_gae(A, B, None, None, None, None, C, None, 4, 4, g, l, S) == ERR_PARAM
    assert lib.rlscan_td_lambda(A, B, None, None, None, None, C, 4, 4, g, l, S) == ERR_PARAM
    assert lib.rlscan_eligibility_traces(A, None, None, None, C, 4, 4, g, l, S) == ERR_PARAM
    assert lib.rlscan_retrace(A, B, C, D, F, None, None, None, None, G, 4, 4, g, l, S) == ERR_PARAM


@pytest.mark.parametrize("rho,c", [(0.0, 1.0), (1.0, -1.0), (math.inf, 1.0), (1.0, math.nan)])
def test_vtrace_clip_errors(lib, rho, c):
    assert lib.rlscan_vtrace(A, B, C, None, None, None, None, D, None, 4, 4, 0.99, 1.0, rho, c, S) == ERR_PARAM


def test_discounted_gamma_range(lib):
    assert lib.rlscan_discounted_returns(A, None, None, None, None, C, 4, 4, 1.0001, S) == ERR_PARAM


def test_null_required_pointers(lib):
    assert lib.rlscan_discounted_returns(None, None, None, None, None, C, 4, 4, 0.99, S) == ERR_NULL
    assert lib.rlscan_discounted_returns(A, None, None, None, None, None, 4, 4, 0.99, S) == ERR_NULL
    assert lib.rlscan_td_lambda(A, None, None, None, None, None, C, 4, 4, 0.99, 0.9, S) == ERR_NULL
    assert lib.rlscan_gae(A, B, None, None, None, None, None, None, 4, 4, 0.99, 0.95, S) == ERR_NULL
    assert lib.rlscan_vtrace(A, B, None, None, None, None, None, D, None, 4, 4, 0.99, 1.0, 1.0, 1.0, S) == ERR_NULL
    assert lib.rlscan_retrace(A, B, C, None, F, None, None, None, None, G, 4, 4, 0.99, 0.9, S) == ERR_NULL
    assert lib.rlscan_eligibility_traces(None, None, None, None, C, 4, 4, 0.99, 0.9, S) == ERR_NULL
    assert lib.rlscan_episodic_prefix_sum(A, None, None, None, None, 4, 4, S) == ERR_NULL
    assert lib.rlscan_linear_scan(A, None, None, C, 4, 4, 1, S) == ERR_NULL


def test_empty_shapes_are_noops(lib):
    # E*T == 0: OK without touching any pointer (all NULL here)
    assert lib.rlscan_gae(None, None, None, None, None, None, None, None, 0, 128, 0.99, 0.95, S) == OK
    assert lib.rlscan_gae(None, None, None, None, None, None, None, None, 64, 0, 0.99, 0.95, S) == OK
    assert lib.rlscan_retrace(None, None, None, None, None, None, None, None, None, None, 0, 0, 0.9, 0.9, S) == OK
    assert lib.rlscan_episodic_prefix_sum(None, None, None, None, None, 0, 5, S) == OK
    assert lib.rlscan_linear_scan(None, None, None, None, 3, 0, 0, S) == OK
    # ...but shape and parameter checks still come first
    assert lib.rlscan_gae(None, None, None, None, None, None, None, None, 0, 128, 2.0, 0.95, S) == ERR_PARAM


def test_misaligned_float_pointers(lib):
    assert lib.rlscan_gae(A + 2, B, None, None, None, None, C, None, 4, 4, 0.99, 0.95, S) == ERR_ALIGN
    assert lib.rlscan_gae(A, B, None, None, None, None, C + 1, None, 4, 4, 0.99, 0.95, S) == ERR_ALIGN
    assert lib.rlscan_gae(A, B, None, None, D + 3, None, C, None, 4, 4, 0.99, 0.95, S) == ERR_ALIGN
    assert lib.rlscan_linear_scan(A, B, C + 2, D, 4, 4, 1, S) == ERR_ALIGN


def test_overlapping_outputs_are_rejected(lib):
    E, T = 8, 16
    n = 4 * E * T
    # output starts inside rewards
    assert lib.rlscan_gae(A, B, None, None, None, None, A + n - 4, None, E, T, 0.99, 0.95, S) == ERR_ALIAS
    # advantages and returns overlap each other
    assert lib.rlscan_gae(A, B, None, None, None, None, C, C + 64, E, T, 0.99, 0.95, S) == ERR_ALIAS
    # output overlaps a flag array (E*T bytes)
    assert lib.rlscan_discounted_returns(A, D, None, None, None, D + E * T - 4, E, T, 0.9, S) == ERR_ALIAS
    # output overlaps the per-row bootstrap
    assert lib.rlscan_td_lambda(A, B, None, None, F, None, F, E, T, 0.9, 0.9, S) == ERR_ALIAS
    assert lib.rlscan_linear_scan(A, B, None, B, E, T, 1, S) == ERR_ALIAS


def test_returns_and_td_lambda_validation(lib):
    E, T = 8, 16
    n = 4 * E * T
    f = lib.rlscan_returns_and_td_lambda
    assert f(A, B, None, None, None, None, C, D, -1, T, 0.99, 0.9, S) == ERR_SHAPE
    assert f(A, B, None, None, None, None, C, D, E, T, 0.99, 1.5, S) == ERR_PARAM
    assert f(A, B, None, None, None, None, C, None, E, T, 0.99, 0.9, S) == ERR_NULL   # td_returns required
    assert f(A, None, None, None, None, None, C, D, E, T, 0.99, 0.9, S) == ERR_NULL   # values required
    assert f(A, B, None, None, None, None, C, C + n - 4, E, T, 0.99, 0.9, S) == ERR_ALIAS  # outputs overlap
    assert f(A, B, None, None, None, None, C, B, E, T, 0.99, 0.9, S) == ERR_ALIAS  # output over an input
    assert f(A, B + 2, None, None, None, None, C, D, E, T, 0.99, 0.9, S) == ERR_ALIGN
    assert f(None, None, None, None, None, None, None, None, 0, T, 0.99, 0.9, S) == OK


def test_linear_scan_segmented_validation(lib):
    E, T = 8, 16
    f = lib.rlscan_linear_scan_segmented
    assert f(A, B, D, None, C, -1, T, 1, S) == ERR_SHAPE
    assert f(A, None, D, None, C, E, T, 1, S) == ERR_NULL
    assert f(A, B, D, None, None, E, T, 0, S) == ERR_NULL
    assert f(A + 1, B, D, None, C, E, T, 1, S) == ERR_ALIGN
    assert f(A, B, D, None, D + E * T - 4, E, T, 1, S) == ERR_ALIAS  # output over the flags
    assert f(None, None, None, None, None, E, 0, 1, S) == OK


def test_eligibility_traces_vec_validation(lib):
    E, T, Dm = 4, 8, 16
    f = lib.rlscan_eligibility_traces_vec
    assert f(A, None, None, None, C, E, T, -1, 0.9, 0.9, S) == ERR_SHAPE
    assert f(A, None, None, None, C, E, 2 ** 40, 2 ** 40, 0.9, 0.9, S) == ERR_SHAPE
    assert f(A, None, None, None, C, E, T, Dm, 0.9, 1.5, S) == ERR_PARAM
    assert f(None, None, None, None, C, E, T, Dm, 0.9, 0.9, S) == ERR_NULL
    assert f(A, None, None, F + 2, C, E, T, Dm, 0.9, 0.9, S) == ERR_ALIGN
    assert f(A, None, None, None, A + 4 * E * T * Dm - 4, E, T, Dm, 0.9, 0.9, S) == ERR_ALIAS
    assert f(A, D, None, None, D + 8, E, T, Dm, 0.9, 0.9, S) == ERR_ALIAS  # output over the flags
    assert f(None, None, None, None, None, E, T, 0, 0.9, 0.9, S) == OK


F32, BF16, F16 = 0, 1, 2
ENV_MAJOR, TIME_MAJOR = 0, 1


@pytest.mark.parametrize("lay", [ENV_MAJOR, TIME_MAJOR])
def test_ex_entries_validation(lib, lay):
    E, T = 8, 16

    def gae(fmt, *a):
        return lib.rlscan_gae_ex(fmt, lay, *a)

    # unknown storage format or layout
    assert gae(7, A, B, None, None, None, None, C, None, E, T, 0.99, 0.95, S) == ERR_PARAM
    assert gae(-1, A, B, None, None, None, None, C, None, E, T, 0.99, 0.95, S) == ERR_PARAM
    assert lib.rlscan_gae_ex(F32, 2, A, B, None, None, None, None, C, None, E, T, 0.99, 0.95, S) == ERR_PARAM
    assert lib.rlscan_gae_ex(BF16, -1, A, B, None, None, None, None, C, None, E, T, 0.99, 0.95, S) == ERR_PARAM
    for fmt in (BF16, F16):
        # 16-bit storage needs 2-byte alignment only
        assert gae(fmt, A + 1, B, None, None, None, None, C, None, E, T, 0.99, 0.95, S) == ERR_ALIGN
        assert gae(fmt, A, B, None, None, None, None, C + 3, None, E, T, 0.99, 0.95, S) == ERR_ALIGN
        assert gae(fmt, A, B, None, None, F + 1, None, C, None, E, T, 0.99, 0.95, S) == ERR_ALIGN
        # overlap is measured in 2-byte elements: the last element of rewards
        # overlaps, the first byte past it does not (then validation passes and
        # a NULL output is the next error)
        assert gae(fmt, A, B, None, None, None, None, A + 2 * E * T - 2, None, E, T, 0.99, 0.95, S) == ERR_ALIAS
        assert gae(fmt, A, B, None, None, None, None, C, C + 2 * E * T - 2, E, T, 0.99, 0.95, S) == ERR_ALIAS
        assert gae(fmt, A, B, None, None, None, None, None, None, E, T, 0.99, 0.95, S) == ERR_NULL
        assert gae(fmt, A, B, None, None, None, None, C, None, -1, T, 0.99, 0.95, S) == ERR_SHAPE
        assert gae(fmt, A, B, None, None, None, None, C, None, E, T, 0.99, 1.5, S) == ERR_PARAM
        assert gae(fmt, None, None, None, None, None, None, None, None, 0, T, 0.99, 0.95, S) == OK
        assert lib.rlscan_discounted_returns_ex(fmt, lay, None, None, None, None, None, C, E, T, 0.9, S) == ERR_NULL
        assert lib.rlscan_td_lambda_ex(fmt, lay, A, None, None, None, None, None, C, E, T, 0.9, 0.9, S) == ERR_NULL
        assert lib.rlscan_vtrace_ex(fmt, lay, A, B, D, None, None, None, None, C, None, E, T, 0.9, 1.0, 0.0, 1.0,
                                    S) == ERR_PARAM
        assert lib.rlscan_retrace_ex(fmt, lay, A, B, C, D, None, None, None, None, None, F, E, T, 0.9, 0.9,
                                     S) == ERR_NULL
        assert lib.rlscan_eligibility_traces_ex(fmt, lay, A, None, None, F + 1, C, E, T, 0.9, 0.9, S) == ERR_ALIGN
        assert lib.rlscan_episodic_prefix_sum_ex(fmt, lay, A, None, None, None, A + 2, E, T, S) == ERR_ALIAS
    rtx = lib.rlscan_returns_and_td_lambda_ex
    assert rtx(5, lay, A, B, None, None, None, None, C, D, E, T, 0.9, 0.9, S) == ERR_PARAM
    assert rtx(BF16, lay, A, B, None, None, None, None, C, None, E, T, 0.9, 0.9, S) == ERR_NULL
    assert rtx(F16, lay, A + 1, B, None, None, None, None, C, D, E, T, 0.9, 0.9, S) == ERR_ALIGN
    assert rtx(BF16, lay, A, B, None, None, None, None, C, C + 2 * E * T - 2, E, T, 0.9, 0.9, S) == ERR_ALIAS
    tvx = lib.rlscan_eligibility_traces_vec_ex
    assert tvx(4, lay, A, None, None, None, C, E, T, 8, 0.9, 0.9, S) == ERR_PARAM
    assert tvx(BF16, 7, A, None, None, None, C, E, T, 8, 0.9, 0.9, S) == ERR_PARAM
    assert tvx(BF16, lay, A + 1, None, None, None, C, E, T, 8, 0.9, 0.9, S) == ERR_ALIGN
    assert tvx(F16, lay, A, None, None, None, A + 2 * E * T * 8 - 2, E, T, 8, 0.9, 0.9, S) == ERR_ALIAS
    assert tvx(F16, lay, A, None, None, None, C, E, T, -1, 0.9, 0.9, S) == ERR_SHAPE
    assert tvx(BF16, lay, None, None, None, None, None, E, T, 0, 0.9, 0.9, S) == OK
    lsx = lib.rlscan_linear_scan_segmented_ex
    assert lsx(9, lay, A, B, None, None, C, E, T, 1, S) == ERR_PARAM
    assert lsx(BF16, 3, A, B, None, None, C, E, T, 1, S) == ERR_PARAM
    assert lsx(BF16, lay, A + 1, B, None, None, C, E, T, 1, S) == ERR_ALIGN
    assert lsx(F16, lay, A, None, None, None, C, E, T, 0, S) == ERR_NULL
    assert lsx(F16, lay, A, B, D, None, D + E * T - 2, E, T, 0, S) == ERR_ALIAS  # output over the flags
    assert lsx(BF16, lay, None, None, None, None, None, 0, T, 1, S) == OK
    # the float32 format through the _ex entry keeps the 4-byte rules
    assert gae(F32, A + 2, B, None, None, None, None, C, None, E, T, 0.99, 0.95, S) == ERR_ALIGN
    assert gae(F32, A, B, None, None, None, None, A + 4 * E * T - 4, None, E, T, 0.99, 0.95, S) == ERR_ALIAS


def test_binding_rejects_mixed_storage_dtypes():
    torch = pytest.importorskip("torch")
    r = torch.zeros(2, 3, dtype=torch.bfloat16)
    v = torch.zeros(2, 3, dtype=torch.float32)
    with pytest.raises(TypeError, match="values must be bfloat16"):
        rl._check_val(v, "values", (2, 3), v.device, rl._storage(r, "rewards"))
    with pytest.raises(TypeError, match="float32, bfloat16 or float16"):
        rl._storage(torch.zeros(2, 3, dtype=torch.float64), "rewards")


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(rl, "_LIB_PATH", "/nonexistent/librlscan.so")
    monkeypatch.setattr(rl, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        rl.lib()


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    r = torch.zeros(2, 3)
    with pytest.raises(ValueError, match="GPU"):
        rl.discounted_returns(r)


def test_grid_limits_are_shape_errors(lib):
    # launches whose grid would pass 2^32 - 1 work-items are refused in
    # validation (before any HIP call), not at launch time
    tm_max_e = 64 * (0xFFFFFFFF // (64 * 16))  # largest time-major E: one 16-wave block per 64 envs
    for fmt in (F32, BF16):
        big = tm_max_e + 1
        assert lib.rlscan_gae_ex(fmt, TIME_MAJOR, A, B, None, None, None, None, C, None, big, 1, 0.99, 0.95,
                                 S) == ERR_SHAPE
        assert lib.rlscan_discounted_returns_ex(fmt, TIME_MAJOR, A, None, None, None, None, C, big, 2, 0.9,
                                                S) == ERR_SHAPE
        assert lib.rlscan_retrace_ex(fmt, TIME_MAJOR, A, B, C, D, F, None, None, None, None, G, big, 1, 0.9, 0.9,
                                     S) == ERR_SHAPE
        assert lib.rlscan_linear_scan_segmented_ex(fmt, TIME_MAJOR, A, B, None, None, C, big, 1, 1, S) == ERR_SHAPE
        assert lib.rlscan_returns_and_td_lambda_ex(fmt, TIME_MAJOR, A, B, None, None, None, None, C, D, big, 1,
                                                   0.9, 0.9, S) == ERR_SHAPE
        # at the limit itself validation passes: with NULL outputs the next error is ERR_NULL
        assert lib.rlscan_gae_ex(fmt, TIME_MAJOR, A, B, None, None, None, None, None, None, tm_max_e, 1, 0.99,
                                 0.95, S) == ERR_NULL
        # the same E row-major is not limited by this grid
        assert lib.rlscan_gae_ex(fmt, ENV_MAJOR, A, B, None, None, None, None, None, None, big, 1, 0.99, 0.95,
                                 S) == ERR_NULL
    # vector traces: one 4-wave block per row and 64 feature columns
    tv_max_blocks = 0xFFFFFFFF // (64 * 4)
    f = lib.rlscan_eligibility_traces_vec
    assert f(A, None, None, None, C, tv_max_blocks + 1, 1, 64, 0.9, 0.9, S) == ERR_SHAPE
    assert f(A, None, None, None, C, tv_max_blocks // 2 + 1, 1, 65, 0.9, 0.9, S) == ERR_SHAPE
    assert f(A, None, None, None, None, tv_max_blocks, 1, 64, 0.9, 0.9, S) == ERR_NULL
    assert lib.rlscan_eligibility_traces_vec_ex(BF16, TIME_MAJOR, A, None, None, None, C, tv_max_blocks + 1, 1, 64,
                                                0.9, 0.9, S) == ERR_SHAPE
