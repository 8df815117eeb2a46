"""The bench's agreement fields (CPU): outputs equal to the oracle's rounded to
float32 pass the gate; an output off by 2e-5 (relative where |ref| >= 1,
absolute below) fails it; 16-bit storage widens the gate by the format's unit
roundoff."""
from __future__ import annotations

import dataclasses

import numpy as np

import bench
from linear_recurrence_scan_reverse_amd import synth


def _small():
    w = dataclasses.replace(synth.WORKLOADS["all7_16384x256"], E=32, T=64)
    return w, synth.workload_inputs(w)


def _rounded_reference(w, d, names):
    return {n: {k: v.astype(np.float32) for k, v in bench.oracle_reference(n, d, w).items()} for n in names}


def test_rounded_oracle_outputs_pass():
    w, d = _small()
    names = list(bench.ORDER) + ["returns_and_td_lambda", "linear_scan_segmented"]
    res = bench.agreement_of(_rounded_reference(w, d, names), d, w, "f32")
    assert set(res) >= {"vtrace", "vtrace.out1", "returns_and_td_lambda.out1", "linear_scan_segmented"}
    for k, v in res.items():
        assert v["pass"] and v["max_err"] <= 2.0 ** -24, (k, v)
        assert v["max_abs_ref"] > 0


def test_an_error_past_the_gate_fails():
    w, d = _small()
    gpu = _rounded_reference(w, d, ["retrace"])
    ref = bench.oracle_reference("retrace", d, w)["out"]
    i = np.unravel_index(np.argmax(np.abs(ref)), ref.shape)
    bad = gpu["retrace"]["out"].astype(np.float64)
    bad[i] += 2e-5 * max(1.0, abs(ref[i]))
    gpu["retrace"]["out"] = bad.astype(np.float32)
    res = bench.agreement_of(gpu, d, w, "f32")
    assert not res["retrace"]["pass"]
    assert res["retrace"]["max_err"] > bench.TOL
    # the same error is inside the bfloat16 gate
    assert bench.agreement_of(gpu, d, w, "bf16")["retrace"]["pass"]


def test_kernel_trace_summary_needs_matching_sources(tmp_path, monkeypatch):
    path = tmp_path / "kernel_trace_rlscan_demo.txt"
    path.write_text("# kernel_source_sha256: %s\nretrace  scan_kernel<Retrace>  calls 200  avg 19.50  min 19.0\n"
                    % bench.kernel_source_hash())
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    us, src = bench.read_kernel_us("retrace", "demo")
    assert us == 19.5
    path.write_text("# kernel_source_sha256: 0000\nretrace  k  calls 200  avg 19.50\n")
    us, why = bench.read_kernel_us("retrace", "demo")
    assert us is None and "changed" in why
