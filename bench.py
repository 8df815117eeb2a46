"""Benchmark: RL credit-assignment scans on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of all seven estimators (discounted returns, TD(lambda),
GAE, V-trace vs + pg, Retrace, eligibility traces, episodic prefix sums) over
one synthetic rollout batch of E = 16384 envs x T = 256 steps, each estimator
one call (one kernel) through the C ABI, back to back on one stream.  Inputs are resident in HBM before the
timed region.  To keep the 256 MB Infinity Cache from serving repeat reads,
calls rotate through buffer sets totalling > 1 GiB, so every launch reads cold
data.

Printed (one JSON line on stdout):
  value          env-steps/s through the whole seven-estimator step
  per_estimator  back-to-back launch time of each estimator (200 calls or
                 more), env-steps/s, algorithmic GB/s and fraction of the
                 8 TB/s HBM peak
  roofline       the same for the dominant (slowest) kernel, plus its kernel
                 time and the HBM traffic rocprofv3 recorded for it (when the
                 committed summaries match the current kernel sources)
  cpu_baseline   the fp64 CPU oracle on a bounded sample of the same workload
  agreement      every output of the run (the seven estimators, the one-pass
                 entries, the storage formats and layouts, the smaller
                 workloads) against the oracle on the same inputs:
                 max |gpu - oracle| / max(1, |oracle|) and max |oracle|; the
                 line is marked failed (exit status 3) past the gate
  formats_and_layouts  the seven estimators with bfloat16 / float16 value
                 storage and in the time-major [T, E] layout (the _ex
                 entries), same workload, not part of the step
  configs        the four smaller workloads (latency and env-steps/s)
Context only (not comparable): the rl-triton pages report 1.6-5.70x full-call
speedups over a vectorized torch.compile scan on NVIDIA GPUs (H100 80GB HBM3
and RTX 2000 Ada per the gist.science summary; the abstract does not name them).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from linear_recurrence_scan_reverse_amd import synth  # noqa: E402

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
ORDER = ("discounted_returns", "td_lambda", "gae", "vtrace", "retrace",
         "eligibility_traces", "episodic_prefix_sum")
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "linear_recurrence_scan_reverse_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the sources that decide what the kernels do and how they are launched
    (the argument-checking C-ABI file is left out)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".h")) and name != "rlscan_api.hip":
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------- algorithmic bytes
def alg_bytes(name, d, E, T, with_flags=True, vb=4):
    """Bytes the method itself must move for one call: every dense input read once,
    every output written once, [E] arrays once per row, the truncation bootstrap
    only where a step is truncated and not terminated (vb bytes per value)."""
    n = E * T
    f = vb * n
    flags = n * (int("terminated" in d) + int("truncated" in d)) if with_flags else 0
    sparse = 0
    if with_flags and "truncated" in d:
        tb_steps = int(np.count_nonzero(d["truncated"] & (d["terminated"] == 0)))
        sparse = vb * tb_steps
    row = vb * E
    table = {
        "discounted_returns": f + flags + sparse + row + f,
        "td_lambda": 2 * f + flags + sparse + row + f,
        "gae": 2 * f + flags + sparse + row + f,
        "vtrace": 3 * f + flags + sparse + row + 2 * f,
        "retrace": 5 * f + flags + sparse + row + f,
        "eligibility_traces": f + flags + row + f,
        "episodic_prefix_sum": f + flags + row + f,
        "returns_and_td_lambda": 2 * f + flags + sparse + row + 2 * f,
        "linear_scan_segmented": 2 * f + (n if "terminated" in d else 0) + f,
    }
    return table[name]


# ----------------------------------------------------------------- GPU side
# storage formats of the _ex entries (rlscan_format) and their value dtypes
FORMATS = {"f32": (0, "float32"), "bf16": (1, "bfloat16"), "f16": (2, "float16")}
VALUE_KEYS = ("r", "v", "log_rhos", "q", "exp_q", "pi", "mu", "bootstrap_value", "trunc_bootstrap")
ROW_KEYS = ("bootstrap_value",)


class _Ex:
    """The library with every estimator entry bound to one storage format and layout."""

    def __init__(self, lib, fmt, layout):
        self._lib, self._fmt, self._layout = lib, fmt, layout

    def __getattr__(self, name):
        fn = getattr(self._lib, name + "_ex")
        return lambda *a: fn(self._fmt, self._layout, *a)


class Runner:
    """Pre-resolved C-ABI calls over rotating device buffer sets."""

    def __init__(self, w, d, nsets, device, storage="f32", time_major=False):
        import torch
        import linear_recurrence_scan_reverse_amd as rl

        self.torch = torch
        fmt, dname = FORMATS[storage]
        vdt = getattr(torch, dname)
        self.vb = torch.empty(0, dtype=vdt).element_size()
        self.lib = rl.lib() if (fmt == 0 and not time_major) else _Ex(rl.lib(), fmt, 1 if time_major else 0)
        self.E, self.T = w.E, w.T
        self.w = w
        self.time_major = time_major
        self.stream = torch.cuda.current_stream(device)
        self.sptr = self.stream.cuda_stream
        base = {k: torch.from_numpy(np.ascontiguousarray(v)).to(device) for k, v in d.items()}
        base = {k: (v.to(vdt) if k in VALUE_KEYS else v) for k, v in base.items()}
        # the values the kernels read, widened back to float32 (the oracle's inputs)
        self.host_inputs = {k: (v.float().cpu().numpy() if k in VALUE_KEYS else d[k]) for k, v in base.items()}
        if time_major:  # [T, E] per-step arrays (E and T keep their meaning)
            base = {k: (v if k in ROW_KEYS else v.t().contiguous()) for k, v in base.items()}
        self.sets = []
        for i in range(nsets):
            s = {k: (v if i == 0 else v.clone()) for k, v in base.items()}
            for o in ORDER:
                s["out_" + o] = torch.empty((w.E, w.T), dtype=vdt, device=device)
            s["out_vtrace_pg"] = torch.empty((w.E, w.T), dtype=vdt, device=device)
            ptrs = {k: None for k in ("terminated", "truncated", "bootstrap_value", "trunc_bootstrap")}
            ptrs.update({k: v.data_ptr() for k, v in s.items()})
            self.sets.append(ptrs)
            self.sets[-1]["_keep"] = s
        self.set_bytes = sum(v.numel() * v.element_size() for v in self.sets[0]["_keep"].values())
        self.counter = 0

    def call(self, name, s):
        L, E, T, w, st = self.lib, self.E, self.T, self.w, self.sptr
        p = s
        if name == "discounted_returns":
            rc = L.rlscan_discounted_returns(p["r"], p["terminated"], p["truncated"], p["bootstrap_value"],
                                             p["trunc_bootstrap"], p["out_" + name], E, T, w.gamma, st)
        elif name == "td_lambda":
            rc = L.rlscan_td_lambda(p["r"], p["v"], p["terminated"], p["truncated"], p["bootstrap_value"],
                                    p["trunc_bootstrap"], p["out_" + name], E, T, w.gamma, w.lam, st)
        elif name == "returns_and_td_lambda":
            rc = L.rlscan_returns_and_td_lambda(p["r"], p["v"], p["terminated"], p["truncated"],
                                                p["bootstrap_value"], p["trunc_bootstrap"],
                                                p["out_discounted_returns"], p["out_td_lambda"], E, T,
                                                w.gamma, w.lam, st)
        elif name == "linear_scan_segmented":
            # the generic episode-cut recurrence: a = pi (in (0.05, 1)), b = r, cuts at terminations
            rc = L.rlscan_linear_scan_segmented(p["pi"], p["r"], p["terminated"], None,
                                                p["out_episodic_prefix_sum"], E, T, 1, st)
        elif name == "gae":
            rc = L.rlscan_gae(p["r"], p["v"], p["terminated"], p["truncated"], p["bootstrap_value"],
                              p["trunc_bootstrap"], p["out_" + name], None, E, T, w.gamma, w.lam, st)
        elif name == "vtrace":
            rc = L.rlscan_vtrace(p["r"], p["v"], p["log_rhos"], p["terminated"], p["truncated"],
                                 p["bootstrap_value"], p["trunc_bootstrap"], p["out_" + name],
                                 p["out_vtrace_pg"], E, T, w.gamma, w.vtrace_lam, w.rho_bar, w.c_bar, st)
        elif name == "retrace":
            rc = L.rlscan_retrace(p["r"], p["q"], p["exp_q"], p["pi"], p["mu"], p["terminated"],
                                  p["truncated"], p["bootstrap_value"], p["trunc_bootstrap"],
                                  p["out_" + name], E, T, w.gamma, w.lam, st)
        elif name == "eligibility_traces":
            rc = L.rlscan_eligibility_traces(p["r"], p["terminated"], p["truncated"], p["bootstrap_value"],
                                             p["out_" + name], E, T, w.gamma, w.lam, st)
        elif name == "episodic_prefix_sum":
            rc = L.rlscan_episodic_prefix_sum(p["r"], p["terminated"], p["truncated"], p["bootstrap_value"],
                                              p["out_" + name], E, T, st)
        else:
            raise KeyError(name)
        if rc != 0:
            raise RuntimeError("%s returned status %d" % (name, rc))

    # output tensors each entry writes, by output key
    OUTPUTS = {"vtrace": {"out": "out_vtrace", "out1": "out_vtrace_pg"},
               "returns_and_td_lambda": {"out": "out_discounted_returns", "out1": "out_td_lambda"},
               "linear_scan_segmented": {"out": "out_episodic_prefix_sum"}}

    def outputs(self, name):
        """One call of an entry on buffer set 0, its outputs copied to the host as
        float32 [E, T] numpy arrays."""
        torch = self.torch
        s = self.sets[0]
        self.call(name, s)
        torch.cuda.synchronize()
        res = {}
        for k, key in self.OUTPUTS.get(name, {"out": "out_" + name}).items():
            t = s["_keep"][key]
            if self.time_major:
                t = t.view(self.T, self.E).t()
            res[k] = t.float().cpu().numpy()
        return res

    def next_set(self):
        s = self.sets[self.counter % len(self.sets)]
        self.counter += 1
        return s

    def step(self, names):
        for n in names:
            self.call(n, self.next_set())


def time_region(runner, fn, reps):
    torch = runner.torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(runner.stream)
    for _ in range(reps):
        fn()
    end.record(runner.stream)
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3  # seconds


# Arrays one estimator call streams per step: float32 inputs, one-byte flag
# arrays, float32 outputs.  The [E] row values and the sparse truncation
# bootstraps are left out (under 0.2% of the bytes at 256 steps).
PROBE_MIX = {
    "discounted_returns": (1, 2, 1), "td_lambda": (2, 2, 1), "gae": (2, 2, 1), "vtrace": (3, 2, 2),
    "retrace": (5, 2, 1), "eligibility_traces": (1, 2, 1), "episodic_prefix_sum": (1, 2, 1),
    "returns_and_td_lambda": (2, 2, 2), "linear_scan_segmented": (2, 1, 1),
}
PROBE_LIB = os.path.join(ROOT, "linear_recurrence_scan_reverse_amd", "libstreamprobe.so")
PROBE_SHAPES = ("grid16", "grid32", "grid64", "grid16w", "persist", "grid32w")
_probe = None


def probe_lib():
    """libstreamprobe.so with argument types set, or None when it is not built."""
    global _probe
    import ctypes
    if _probe is None and os.path.exists(PROBE_LIB):
        lib = ctypes.CDLL(PROBE_LIB)
        P = ctypes.POINTER(ctypes.c_void_p)
        lib.stream_probe_time.restype = ctypes.c_int
        lib.stream_probe_time.argtypes = [P, ctypes.c_int, P, ctypes.c_int, P, ctypes.c_int, ctypes.c_int64,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.POINTER(ctypes.c_float)]
        lib.stream_probe_shapes.restype = ctypes.c_int
        assert lib.stream_probe_shapes() == len(PROBE_SHAPES)
        _probe = lib
    return _probe


def probe_sweep(torch, device, n, mix, reps=200, nsets=None, shapes=None):
    """Per-launch us of every plain streaming shape (libstreamprobe.so) moving one
    call's arrays (mix = float inputs, flag arrays, float outputs; n elements
    each), over rotating buffer sets above 1 GiB, timed in the probe library with
    HIP events on the launch stream: {shape name: us}, or None when the probe
    library is not built."""
    import ctypes
    lib = probe_lib()
    if lib is None:
        return None
    nr, nf, nw = mix
    set_bytes = n * (4 * nr + nf + 4 * nw)
    nsets = nsets or int(min(64, max(2, -(-(1 << 30) // set_bytes) + 1)))
    keep, ins, fls, outs = [], [], [], []
    for _ in range(nsets):
        i_ = [torch.ones(n, dtype=torch.float32, device=device) for _ in range(nr)]
        f_ = [torch.zeros(n, dtype=torch.uint8, device=device) for _ in range(nf)]
        o_ = [torch.empty(n, dtype=torch.float32, device=device) for _ in range(nw)]
        keep.append((i_, f_, o_))
        ins += [t.data_ptr() for t in i_]
        fls += [t.data_ptr() for t in f_]
        outs += [t.data_ptr() for t in o_]
    st = torch.cuda.current_stream(device)
    pi = (ctypes.c_void_p * len(ins))(*ins)
    pf = (ctypes.c_void_p * max(1, len(fls)))(*fls) if fls else None
    po = (ctypes.c_void_p * len(outs))(*outs)
    res = {}
    for k in (shapes if shapes is not None else range(len(PROBE_SHAPES))):
        us = ctypes.c_float(0.0)
        rc = lib.stream_probe_time(pi, nr, pf, nf, po, nw, n, nsets, k, reps, ctypes.c_void_p(st.cuda_stream),
                                   ctypes.byref(us))
        if rc != 0:
            raise RuntimeError("stream_probe_time failed with %d" % rc)
        res[PROBE_SHAPES[k]] = round(us.value, 3)
    del keep
    torch.cuda.synchronize()
    return res


def ceiling_of(sweep):
    """The fastest shape of a probe sweep: (name, us)."""
    k = min(sweep, key=sweep.get)
    return k, sweep[k]


def read_traffic(est, workload):
    """HBM bytes per launch of one estimator's kernel from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE, scaled by a calibration copy), or None
    when the summary is missing or was taken on other kernel sources."""
    path = os.path.join(PROFILES, "hbm_traffic_rlscan_%s.txt" % workload)
    if not os.path.exists(path):
        return None, "no counter summary"
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None, "kernel sources changed since the counters were taken"
    try:
        return float(vals["%s.hbm_bytes_per_launch" % est]), os.path.relpath(path, ROOT)
    except (KeyError, ValueError):
        return None, "malformed counter summary"


def read_kernel_us(est, workload):
    """Average kernel duration (us) of one estimator's back-to-back launches from the
    committed rocprofv3 kernel-trace summary, or None when the summary is missing or
    was taken on other kernel sources."""
    path = os.path.join(PROFILES, "kernel_trace_rlscan_%s.txt" % workload)
    if not os.path.exists(path):
        return None, "no kernel-trace summary"
    rows, sha = {}, None
    with open(path) as f:
        for line in f:
            if line.startswith("# kernel_source_sha256:"):
                sha = line.split(":", 1)[1].strip()
            elif line.strip() and not line.startswith("#"):
                tok = line.split()
                if "avg" in tok:
                    rows[tok[0]] = float(tok[tok.index("avg") + 1])
    if sha != kernel_source_hash():
        return None, "kernel sources changed since the kernel trace was taken"
    if est not in rows:
        return None, "estimator not in the kernel-trace summary"
    return rows[est], os.path.relpath(path, ROOT)


# ----------------------------------------------------------------- the oracle leg (CPU baseline)
# The only part of the bench that runs the oracle: it times the unchanged fp64
# oracle on the host cores (cpu_baseline), and its outputs on the inputs each GPU
# call read are the reference of the agreement fields.
TOL = 1e-5  # max |gpu - oracle| / max(1, |oracle|): relative where |oracle| >= 1, absolute below
UNIT_ROUNDOFF = {"f32": 0.0, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}  # last rounding to the storage format


def oracle_reference(name, d, w):
    """The oracle's outputs of one GPU entry on host inputs d: {output: float64 array}."""
    import oracle

    te, tr = d.get("terminated"), d.get("truncated")
    bv, tb = d.get("bootstrap_value"), d.get("trunc_bootstrap")
    g, lam = w.gamma, w.lam
    if name == "discounted_returns":
        return {"out": oracle.discounted_returns(d["r"], te, tr, bv, tb, gamma=g)}
    if name == "td_lambda":
        return {"out": oracle.td_lambda(d["r"], d["v"], te, tr, bv, tb, gamma=g, lam=lam)}
    if name == "returns_and_td_lambda":
        return {"out": oracle.discounted_returns(d["r"], te, tr, bv, tb, gamma=g),
                "out1": oracle.td_lambda(d["r"], d["v"], te, tr, bv, tb, gamma=g, lam=lam)}
    if name == "gae":
        return {"out": oracle.gae(d["r"], d["v"], te, tr, bv, tb, gamma=g, lam=lam)}
    if name == "vtrace":
        vs, pg = oracle.vtrace(d["r"], d["v"], d["log_rhos"], te, tr, bv, tb, gamma=g, lam=w.vtrace_lam,
                               rho_bar=w.rho_bar, c_bar=w.c_bar)
        return {"out": vs, "out1": pg}
    if name == "retrace":
        return {"out": oracle.retrace(d["r"], d["q"], d["exp_q"], d["pi"], d["mu"], te, tr, bv, tb,
                                      gamma=g, lam=lam)}
    if name == "eligibility_traces":
        return {"out": oracle.eligibility_traces(d["r"], te, tr, bv, gamma=g, lam=lam)}
    if name == "episodic_prefix_sum":
        return {"out": oracle.episodic_prefix_sum(d["r"], te, tr, bv)}
    if name == "linear_scan_segmented":
        return {"out": oracle.linear_scan_segmented(d["pi"], d["r"], te, None, reverse=True)}
    raise KeyError(name)


def agreement_of(gpu, d, w, fmt):
    """Each output of each GPU entry (gpu: {name: {output: host array}}) against the
    oracle on the same host inputs; gate TOL plus the storage format's last rounding."""
    gate = TOL + UNIT_ROUNDOFF[fmt]
    res = {}
    for name, outs in gpu.items():
        ref = oracle_reference(name, d, w)
        for k, got in outs.items():
            r = ref[k]
            err = float(np.max(np.abs(got.astype(np.float64) - r) / np.maximum(1.0, np.abs(r)))) if r.size else 0.0
            res[name if k == "out" else name + "." + k] = {
                "max_err": err, "max_abs_ref": float(np.max(np.abs(r))) if r.size else 0.0,
                "gate": gate, "pass": err <= gate}
    return res


def cpu_baseline(w, d, budget_s=10.0):
    """The fp64 oracle as it stands, all seven estimators, on a row sample."""
    threads = max(1, min(16, len(os.sched_getaffinity(0))))

    def run_rows(lo, hi):
        sl = {k: (v[lo:hi] if v.ndim >= 1 else v) for k, v in d.items()}
        for n in ORDER:
            oracle_reference(n, sl, w)

    # single-thread rate on one 256-row block (also warms the oracle library)
    t0 = time.perf_counter()
    run_rows(0, min(256, w.E))
    single = min(256, w.E) * w.T / (time.perf_counter() - t0)

    # then every thread walks its own block of rows, 256 rows per call, until the deadline
    block = -(-w.E // threads)
    done = [0] * threads
    deadline = time.perf_counter() + budget_s

    def worker(k):
        lo0, hi0 = k * block, min(w.E, (k + 1) * block)
        lo = lo0
        while time.perf_counter() < deadline and hi0 > lo0:
            hi = min(lo + 256, hi0)
            run_rows(lo, hi)
            done[k] += hi - lo
            lo = lo0 if hi >= hi0 else hi

    ths = [threading.Thread(target=worker, args=(k,)) for k in range(threads)]
    t0 = time.perf_counter()
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    secs = time.perf_counter() - t0
    rows = sum(done)
    return {
        "value": rows * w.T / secs,
        "unit": "env-steps/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d env rows x %d steps (repeated passes over the %d-row workload), all seven "
                  "estimators, fp64 C oracle (gcc -O2), %d threads over row blocks, %.1f s"
                  % (rows, w.T, w.E, threads, secs),
        "single_thread_env_steps_per_s": single,
        "host": host_info(),
    }


def host_info():
    """CPU count, affinity-limited count and model of the host the oracle ran on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "model": model}


# ----------------------------------------------------------------- profile summaries
# The rocprofv3 runs behind the summaries under profiles/, and the summaries
# themselves (written from the runs' CSV output; no GPU needed):
#   python3 bench.py --profile-commands OUT > run.sh   (then: bash run.sh)
#   python3 bench.py --summarize OUT                   (writes profiles/*.txt)
# A main run's per-estimator timing is 200 or more back-to-back calls of one
# kernel; the summaries average each estimator's kernel over the longest such
# run of consecutive dispatches, so warm-up and step calls do not enter.
PROFILE_MAIN = {  # main runs profiled: name -> bench.py arguments
    "f32": [],
    "bf16": ["--storage", "bf16"],
    "tm_f32": ["--time-major"],
}
PMC_PASSES = {  # one rocprofv3 --pmc run each (within the per-block counter limits)
    "A": "SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
         "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_VMEM GRBM_GUI_ACTIVE",
    "B": "SQ_INSTS_VALU SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_SMEM "
         "SQ_ACTIVE_INST_LDS SQ_WAVES GRBM_GUI_ACTIVE",
    "C": "TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum TCC_EA0_WRREQ_sum",
    "F": "FETCH_SIZE",
    "W": "WRITE_SIZE",
}
PROFILE_RUN_ARGS = ["--steps", "2", "--warmup", "1", "--no-cpu", "--no-ceiling", "--no-16", "--no-configs"]
KERNEL_TAGS = {"DiscountedReturn": "discounted_returns", "TdLambda": "td_lambda", "Gae": "gae", "Vtrace": "vtrace",
               "Retrace": "retrace", "EligibilityTrace": "eligibility_traces",
               "EpisodicPrefixSum": "episodic_prefix_sum", "ReturnsTdLambda": "returns_and_td_lambda"}
CLOCK_GHZ = 2.4   # MI355X peak engine clock
SIMDS = 256 * 4   # compute units x SIMDs


def profile_commands(out):
    """Shell commands (one GPU step each, bounded) that produce every rocprofv3
    output the summaries read, under directory `out`."""
    bench = os.path.join(ROOT, "bench.py")
    run = "python3 %s --steps 5 --warmup 2 --no-cpu --no-configs --no-ceiling" % bench
    lines = ["set -o pipefail", "cd /tmp && export TMPDIR=/tmp", "mkdir -p %s" % out,
             "timeout -k 10 600 %s > %s/bench_plain.json" % (run, out),
             "timeout -k 10 600 rocprofv3 --kernel-trace --stats --output-format csv -d %s/kt -o kt -- %s > "
             "%s/bench.json" % (out, run, out)]
    for m, extra in PROFILE_MAIN.items():
        for ps, counters in PMC_PASSES.items():
            lines.append("timeout -s KILL 180 rocprofv3 --pmc %s --output-format csv -d %s/pmc/%s/%s -o pmc -- "
                         "python3 %s %s" % (counters, out, m, ps, bench, " ".join(PROFILE_RUN_ARGS + extra)))
    for ps in ("F", "W"):
        lines.append("timeout -s KILL 120 rocprofv3 --pmc %s --output-format csv -d %s/cal/%s -o pmc -- "
                     "python3 %s --calibration-copy" % (PMC_PASSES[ps], out, ps, bench))
    return "\n".join(l + (" &&" if i < len(lines) - 1 and i >= 1 else "") for i, l in enumerate(lines))


def _kernel_short(name):
    """A kernel's name without return type, namespace and argument list."""
    name = name.strip().replace("rlscan::", "").replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            name = name[:i]
            break
    return name.strip()


def _read_dispatches(pattern):
    """Dispatches of one rocprofv3 CSV output (kernel trace or counter
    collection): list of {name, us, counters}, in dispatch order."""
    import csv
    import glob
    files = sorted(glob.glob(pattern, recursive=True))
    if len(files) != 1:
        raise SystemExit("expected one file for %s, found %d" % (pattern, len(files)))
    disp = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            k = int(r.get("Dispatch_Id") or r.get("Correlation_Id"))
            e = disp.setdefault(k, {"name": _kernel_short(r["Kernel_Name"]), "counters": {},
                                    "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0})
            if "Counter_Name" in r:
                e["counters"][r["Counter_Name"]] = e["counters"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [disp[k] for k in sorted(disp)]


def _timed_runs(disp, min_len=100):
    """{kernel: dispatches of its longest run of consecutive calls} for runs of
    at least min_len calls (the bench's back-to-back timing)."""
    best, i = {}, 0
    while i < len(disp):
        j = i
        while j < len(disp) and disp[j]["name"] == disp[i]["name"]:
            j += 1
        if j - i >= min_len and j - i > len(best.get(disp[i]["name"], [])):
            best[disp[i]["name"]] = disp[i:j]
        i = j
    return best


def _estimator_of(kernel):
    import re
    m = re.search(r"<(\w+)", kernel)
    return KERNEL_TAGS.get(m.group(1)) if m else None


def _bench_json(path):
    for line in reversed(open(path).read().splitlines()):
        if line.startswith("{"):
            return json.loads(line)
    raise SystemExit("no bench line in %s" % path)


def summarize_profiles(out):
    """Write the profiles/ summaries from the rocprofv3 output under `out`."""
    sha = kernel_source_hash()
    cmd_note = ["# commands (repository root, one MI355X; OUT an empty directory):",
                "#   python3 bench.py --profile-commands OUT > run.sh && bash run.sh",
                "#   python3 bench.py --summarize OUT",
                "# (run.sh: the rocprofv3 runs listed by --profile-commands; each averages an estimator's",
                "#  kernel over its longest run of back-to-back calls, the bench's 200-call timing)"]
    # HIP-event times of an unprofiled run of the same bench command (under the
    # profiler, launches are spaced by its per-dispatch work, so events there
    # time the host, not the kernels)
    bl = _bench_json(os.path.join(out, "bench_plain.json"))
    if bl.get("kernel_source_sha256") != sha or _bench_json(os.path.join(out, "bench.json")).get(
            "kernel_source_sha256") != sha:
        raise SystemExit("the profiled runs used other kernel sources")
    runs = _timed_runs(_read_dispatches(os.path.join(out, "kt", "**", "*kernel_trace.csv")))
    events = {("f32", n): e["us_per_launch"] for n, e in bl["per_estimator"].items()}
    for n, e in (bl.get("one_pass_entries") or {}).items():
        if "us_per_launch" in e:
            events[("f32", n)] = e["us_per_launch"]
    for fmt, per in (bl.get("formats_and_layouts") or {}).items():
        for n, e in per.items():
            events[(fmt, n)] = e["us_per_launch"]

    def fmt_of(k):
        s = "bf16" if "Bf16S" in k else "f16" if "F16S" in k else "f32"
        return ("time_major_" + s) if k.startswith(("tm_kernel", "tm_carry", "tm_item_kernel", "tm_dma_kernel")) else s

    rows = {}
    for k, v in runs.items():
        n = _estimator_of(k)
        if n:
            rows.setdefault(fmt_of(k), []).append((n, k, v))
    head = ["# kernel_source_sha256: %s" % sha,
            "# columns: estimator, kernel (template arguments), calls averaged, average / min / max",
            "#   duration (us), and the per-launch time HIP events measured for the same 200 calls",
            "#   in an unprofiled run of the same command (the bench's timing)"] + cmd_note + [""]
    order = list(ORDER) + ["returns_and_td_lambda"]
    main = ["# rocprofv3 kernel trace: librlscan kernels, workload all7_16384x256 (E=16384, T=256), float32"] + head
    other = ["# rocprofv3 kernel trace: librlscan kernels, workload all7_16384x256 (E=16384, T=256),",
             "# 16-bit storage and the time-major layout (first column: format:estimator)"] + head
    for fmt in ["f32", "bf16", "f16", "time_major_f32", "time_major_bf16"]:
        for n, k, v in sorted(rows.get(fmt, []), key=lambda r: order.index(r[0]) if r[0] in order else 99):
            us = [x["us"] for x in v]
            ev = events.get((fmt, n))
            line = "%-34s %-46s calls %4d  avg %7.2f  min %7.2f  max %7.2f   events %s" % (
                n if fmt == "f32" else "%s:%s" % (fmt, n), k, len(us), sum(us) / len(us), min(us), max(us),
                "%7.2f" % ev if ev else "   -")
            (main if fmt == "f32" else other).append(line)
    wl = "all7_16384x256"
    with open(os.path.join(PROFILES, "kernel_trace_rlscan_%s.txt" % wl), "w") as f:
        f.write("\n".join(main) + "\n")
    with open(os.path.join(PROFILES, "kernel_trace_rlscan_formats_layouts_%s.txt" % wl), "w") as f:
        f.write("\n".join(other) + "\n")

    # counters: calibration (a plain copy of known size) for the traffic counters
    cal = {}
    for ps, cname in (("F", "FETCH_SIZE"), ("W", "WRITE_SIZE")):
        d = [x for x in _read_dispatches(os.path.join(out, "cal", ps, "**", "*counter_collection.csv"))
             if "grid_kernel" in x["name"]]
        cal[ps] = sum(x["counters"][cname] for x in d) / len(d)
    moved_kib = float(1 << 20)  # the calibration copy reads and writes 1 GiB per launch
    scale = {"F": moved_kib / cal["F"], "W": moved_kib / cal["W"]}

    w = synth.WORKLOADS[wl]
    d = synth.workload_inputs(w)
    traffic = ["# HBM traffic per launch of the librlscan kernels, workload %s (E=%d, T=%d), float32" % (wl, w.E, w.T),
               "# hbm bytes = FETCH_SIZE * 1024 * read_scale + WRITE_SIZE * 1024 * write_scale (per-dispatch",
               "#   averages over each estimator's back-to-back calls); the scales make the same counters",
               "#   read 1 GiB each way for a plain copy kernel of 1 GiB (%s KiB fetched, %s KiB written" % (
                   "%.1f" % cal["F"], "%.1f" % cal["W"]),
               "#   per copy launch)"] + cmd_note + [
               "kernel_source_sha256: %s" % sha, "read_scale: %.4f" % scale["F"], "write_scale: %.4f" % scale["W"]]
    ctr = ["# rocprofv3 counters of the librlscan kernels, workload %s (E=%d, T=%d)" % (wl, w.E, w.T),
           "# per launch, averaged over each estimator's back-to-back calls:",
           "#   waves            SQ_WAVES",
           "#   valu/wave ...    SQ_INSTS_VALU, _VMEM_RD, _VMEM_WR, _LDS, _SALU per wave",
           "#   valu_us          SQ_INSTS_VALU x 4 cycles / %d SIMDs / %.1f GHz: the time every SIMD spends" % (
               SIMDS, CLOCK_GHZ),
           "#                    issuing vector instructions if the work spreads evenly (a wave64 VALU",
           "#                    instruction occupies its SIMD for 4 cycles or more)",
           "#   valu_active      SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES: share of resident wave time issuing VALU",
           "#   wait_mem         SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES: share of resident wave time waiting at a",
           "#                    s_waitcnt for memory",
           "#   waves/CU         SQ_WAVE_CYCLES x 4 / (256 CUs x kernel cycles at %.1f GHz): mean resident waves" % CLOCK_GHZ,
           "#   l2_hit           TCC_HIT / (TCC_HIT + TCC_MISS)",
           "#   hbm/alg          HBM bytes (FETCH_SIZE, WRITE_SIZE as in the traffic summary) / algorithmic bytes",
           "# kernel_us is the profiled dispatch duration (counter collection serializes and slows",
           "# dispatches; the kernel-trace summary has the unperturbed times)"] + cmd_note + [
           "kernel_source_sha256: %s" % sha, ""]
    hdr = "%-30s %-44s %6s %7s %6s %6s %6s %6s %7s %7s %7s %7s %7s %7s %7s" % (
        "format:estimator", "kernel", "waves", "valu/w", "vmrd/w", "vmwr/w", "lds/w", "salu/w", "valu_us",
        "valu_act", "wait_mem", "waves/CU", "l2_hit", "hbm/alg", "kernel_us")
    ctr.append(hdr)
    for m in PROFILE_MAIN:
        per_pass = {}
        for ps in PMC_PASSES:
            per_pass[ps] = _timed_runs(_read_dispatches(os.path.join(out, "pmc", m, ps, "**",
                                                                     "*counter_collection.csv")))
        kernels = sorted(set().union(*[set(r) for r in per_pass.values()]))
        vb = 2 if m == "bf16" else 4
        for k in kernels:
            n = _estimator_of(k)
            if not n or n not in ORDER:
                continue

            def avg(ps, c):
                v = per_pass[ps].get(k)
                return sum(x["counters"].get(c, 0.0) for x in v) / len(v) if v else float("nan")
            waves = avg("B", "SQ_WAVES")
            wc = avg("A", "SQ_WAVE_CYCLES")
            durs = [x["us"] for x in per_pass["A"].get(k, [])]
            dur = sum(durs) / len(durs) if durs else float("nan")
            hbm = avg("F", "FETCH_SIZE") * 1024 * scale["F"] + avg("W", "WRITE_SIZE") * 1024 * scale["W"]
            alg = alg_bytes(n, d, w.E, w.T, vb=vb)
            hit, miss = avg("C", "TCC_HIT_sum"), avg("C", "TCC_MISS_sum")
            ctr.append("%-30s %-44s %6d %7.0f %6.1f %6.1f %6.1f %6.0f %7.2f %7.3f %7.3f %7.1f %7.3f %7.3f %7.2f" % (
                "%s:%s" % (m, n), k[:44], waves, avg("B", "SQ_INSTS_VALU") / waves, avg("B", "SQ_INSTS_VMEM_RD") / waves,
                avg("B", "SQ_INSTS_VMEM_WR") / waves, avg("B", "SQ_INSTS_LDS") / waves,
                avg("B", "SQ_INSTS_SALU") / waves, avg("B", "SQ_INSTS_VALU") * 4 / SIMDS / (CLOCK_GHZ * 1e3),
                avg("A", "SQ_ACTIVE_INST_VALU") / wc, avg("A", "SQ_WAIT_INST_ANY") / wc,
                wc * 4 / (256 * dur * CLOCK_GHZ * 1e3), hit / (hit + miss) if hit + miss else float("nan"),
                hbm / alg, dur))
            if m == "f32":
                traffic += ["%s.kernel: %s" % (n, k), "%s.fetch_kib: %.1f" % (n, avg("F", "FETCH_SIZE")),
                            "%s.write_kib: %.1f" % (n, avg("W", "WRITE_SIZE")),
                            "%s.hbm_bytes_per_launch: %d" % (n, round(hbm)),
                            "%s.alg_bytes_per_launch: %d" % (n, alg),
                            "%s.traffic_over_alg: %.3f" % (n, hbm / alg)]
    with open(os.path.join(PROFILES, "hbm_traffic_rlscan_%s.txt" % wl), "w") as f:
        f.write("\n".join(traffic) + "\n")
    with open(os.path.join(PROFILES, "counters_rlscan_%s.txt" % wl), "w") as f:
        f.write("\n".join(ctr) + "\n")
    log("wrote the kernel-trace, traffic and counter summaries under profiles/")


# ----------------------------------------------------------------- main
GRID_E = (256, 1024, 4096, 16384, 65536)
GRID_T = (64, 128, 256, 512, 1024, 2048, 4096)


def drop_truncation(d):
    """The same inputs without per-step truncation (flags and bootstraps absent)."""
    return {k: v for k, v in d.items() if k not in ("truncated", "trunc_bootstrap")}


def add_ceiling(entry, sweep, mix):
    """Attach the probe sweep of an entry's byte mix and its fastest shape."""
    if sweep is None:
        entry["ceiling"] = None
        return
    k, us = ceiling_of(sweep)
    entry["ceiling"] = {"mix": "%d float inputs, %d flag arrays, %d float outputs" % mix, "best_shape": k,
                        "us": us, "frac_of_ceiling": round(us / entry["us_per_launch"], 4), "by_shape": sweep}


def log_estimator(n, e):
    c = e.get("ceiling")
    txt = "  %5.1f%% of the best plain stream of its bytes (%s, %.2f us)" % (
        100 * c["frac_of_ceiling"], c["best_shape"], c["us"]) if c else ""
    log("  %-22s %8.2f us  %7.1f GB/s  %5.1f%% of peak%s" % (
        n, e["us_per_launch"], e["GBps"], 100 * e["frac_of_peak"], txt))


def time_estimators(runner, names, d, w, reps):
    per = {}
    for n in names:
        for _ in range(max(3, len(runner.sets))):  # every buffer set once before timing
            runner.call(n, runner.next_set())
        s = time_region(runner, lambda: runner.call(n, runner.next_set()), reps)
        us = s / reps * 1e6
        b = alg_bytes(n, d, w.E, w.T, vb=runner.vb)
        per[n] = {"us_per_launch": round(us, 3), "env_steps_per_s": w.E * w.T / (us * 1e-6), "alg_bytes": b,
                  "GBps": b / (us * 1e-6) / 1e9, "frac_of_peak": b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
    return per


def time_traces_vec(torch, device, reps, E, T, D, p_term, p_trunc):
    """Per-launch time of the vector traces entry on rotating [E, T, D] buffers."""
    import linear_recurrence_scan_reverse_amd as rl
    f = synth.draw_features(E, T, D, seed=0, p_term=p_term, p_trunc=p_trunc)
    set_bytes = 8 * E * T * D + 2 * E * T + 4 * E * D
    nsets = int(min(16, max(2, -(-(1 << 30) // set_bytes) + 1)))
    base = {k: torch.from_numpy(v).to(device) for k, v in f.items()}
    sets = []
    for i in range(nsets):
        s = {k: (v if i == 0 else v.clone()) for k, v in base.items()}
        s["out"] = torch.empty_like(s["x"])
        sets.append(s)
    lib = rl.lib()
    stream = torch.cuda.current_stream(device)
    st = stream.cuda_stream
    k = [0]

    def call():
        s = sets[k[0] % nsets]
        k[0] += 1
        rc = lib.rlscan_eligibility_traces_vec(s["x"].data_ptr(), s["terminated"].data_ptr(),
                                               s["truncated"].data_ptr(), s["init"].data_ptr(),
                                               s["out"].data_ptr(), E, T, D, 0.99, 0.95, st)
        if rc != 0:
            raise RuntimeError("rlscan_eligibility_traces_vec returned status %d" % rc)

    for _ in range(nsets + 2):
        call()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        call()
    end.record(stream)
    end.synchronize()
    us = start.elapsed_time(end) / reps * 1e3
    b = 8 * E * T * D + 2 * E * T + 4 * E * D
    del sets, base
    return {"shape": "E=%d T=%d D=%d" % (E, T, D), "us_per_launch": round(us, 3), "alg_bytes": b,
            "GBps": b / (us * 1e-6) / 1e9, "frac_of_peak": b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}


def run_grid(torch, device, args):
    """Every estimator over the E x T grid with the all-seven distributions; one
    JSON line per grid point (buffer sets above 1 GiB are skipped)."""
    import dataclasses
    base = synth.WORKLOADS["all7_16384x256"]
    names = list(base.estimators)
    grid_e = [int(x) for x in args.grid_e.split(",")] if args.grid_e else GRID_E
    grid_t = [int(x) for x in args.grid_t.split(",")] if args.grid_t else GRID_T
    st, tm = args.grid_storage, args.grid_time_major
    vb = 2 if st != "f32" else 4
    max_set = int(args.grid_max_gib * (1 << 30))
    for T in grid_t:
        for E in grid_e:
            set_bytes = E * T * (vb * 8 + 2 + vb * 8) + vb * E
            if set_bytes > max_set:
                log("grid %6d x %4d: buffer set %.2f GiB > %g GiB, skipped" % (E, T, set_bytes / 2**30,
                                                                               args.grid_max_gib))
                continue
            w = dataclasses.replace(base, name="all7_%dx%d" % (E, T), E=E, T=T)
            d = synth.workload_inputs(w)
            if args.no_trunc:
                d = drop_truncation(d)
            nsets = int(min(64, max(2, -(-(1 << 30) // set_bytes) + 1)))
            runner = Runner(w, d, nsets, device, storage=st, time_major=tm)
            per = time_estimators(runner, names, d, w, max(200, args.reps))
            log("grid %6d x %4d: " % (E, T) + "  ".join("%s %.2f us %.1f%%" % (
                n[:6], per[n]["us_per_launch"], 100 * per[n]["frac_of_peak"]) for n in names))
            print(json.dumps({"grid": True, "workload": w.name, "E": E, "T": T, "storage": st, "time_major": tm,
                              "truncation": not args.no_trunc, "buffer_sets": nsets,
                              "per_estimator": per}), flush=True)
            del runner
            torch.cuda.empty_cache()


def run_configs(torch, device, args, reps, collect=None):
    """The smaller named workloads (parity cases of the tests), each estimator's
    per-launch time on rotating buffers.  The smallest are cache-resident, so
    their HBM fraction is not meaningful; their figure is latency and
    env-steps/s.  collect: a dict that receives, per workload, the inputs and
    the GPU outputs (for the agreement fields)."""
    res = {}
    for name, w in synth.WORKLOADS.items():
        if name == "all7_16384x256":
            continue
        d = synth.workload_inputs(w)
        set_bytes = sum(v.nbytes for v in d.values()) + 8 * 4 * w.E * w.T
        nsets = int(min(64, max(2, -(-(1 << 30) // set_bytes) + 1)))
        runner = Runner(w, d, nsets, device)
        names = [n for n in ORDER if n in w.estimators]
        per = time_estimators(runner, names, d, w, reps)
        log("config %-18s " % name + "  ".join("%s %.2f us (%.3g env-steps/s)" % (
            n, per[n]["us_per_launch"], per[n]["env_steps_per_s"]) for n in names))
        res[name] = {"E": w.E, "T": w.T, "buffer_sets": nsets, "per_estimator": per}
        if collect is not None:
            collect[name] = (w, d, {n: runner.outputs(n) for n in names})
        del runner
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=200, help="back-to-back calls timed per estimator (at least 200)")
    ap.add_argument("--workload", default="all7_16384x256", choices=list(synth.WORKLOADS))
    ap.add_argument("--only", default=None, help="run only this estimator (profiling)")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets (0 = enough for > 1 GiB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle (baseline and agreement)")
    ap.add_argument("--grid", action="store_true", help="every estimator over the E x T grid, one line each")
    ap.add_argument("--no-trunc", action="store_true", help="inputs without per-step truncation")
    ap.add_argument("--grid-e", default=None, help="comma-separated E values for --grid")
    ap.add_argument("--grid-t", default=None, help="comma-separated T values for --grid")
    ap.add_argument("--no-16", action="store_true", help="skip the 16-bit storage and time-major timings")
    ap.add_argument("--no-configs", action="store_true", help="skip the smaller named workloads")
    ap.add_argument("--configs", action="store_true", help="only the smaller named workloads, one line each")
    ap.add_argument("--grid-storage", default="f32", choices=list(FORMATS), help="value storage for --grid")
    ap.add_argument("--grid-time-major", action="store_true", help="time-major [T, E] arrays for --grid")
    ap.add_argument("--grid-max-gib", type=float, default=1.0, help="largest buffer set --grid runs (GiB)")
    ap.add_argument("--storage", default="f32", choices=list(FORMATS),
                    help="value storage of the main run (profiling one format; the line's value is float32)")
    ap.add_argument("--time-major", action="store_true", help="time-major [T, E] arrays in the main run (profiling)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the plain-stream ceiling sweep (profiling)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="only the counter calibration: the stream probe copying 1 GiB to 1 GiB, 5 times")
    ap.add_argument("--profile-commands", metavar="OUT", default=None,
                    help="print the rocprofv3 runs behind the profiles/ summaries (output under OUT)")
    ap.add_argument("--summarize", metavar="OUT", default=None,
                    help="write the profiles/ summaries from the rocprofv3 output under OUT (no GPU)")
    args = ap.parse_args()
    reps = max(200, args.reps)
    if args.profile_commands:
        print(profile_commands(os.path.abspath(args.profile_commands)))
        return
    if args.summarize:
        summarize_profiles(os.path.abspath(args.summarize))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        log("bench.py: this build measures one GPU only (rows are independent; multi-GPU "
            "sharding is a design note, not implemented). Run with --gpus 1.")
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        log("bench.py: no GPU visible")
        sys.exit(1)
    device = torch.device("cuda", 0)
    torch.cuda.set_device(device)

    if args.calibration_copy:
        us = probe_sweep(torch, device, 1 << 28, (1, 0, 1), reps=5, nsets=2, shapes=[0])["grid16"]
        log("calibration copy: 1 GiB read + 1 GiB written per launch, %.1f us (%.1f GB/s)" % (us, 2**31 / us / 1e3))
        return

    if args.grid:
        run_grid(torch, device, args)
        return

    if args.configs:
        for name, r in run_configs(torch, device, args, reps).items():
            print(json.dumps({"config": True, "workload": name, **r}), flush=True)
        return

    w = synth.WORKLOADS[args.workload]
    names = [n for n in ORDER if n in w.estimators]
    if args.only:
        if args.only not in names:
            raise SystemExit("--only must be one of %s" % names)
        names = [args.only]
    log("workload %s: E=%d T=%d estimators=%s" % (w.name, w.E, w.T, ",".join(names)))
    d = synth.workload_inputs(w)
    if args.no_trunc:
        d = drop_truncation(d)
    set_bytes_est = sum(v.nbytes for v in d.values()) + 8 * 4 * w.E * w.T
    main_vb = 2 if args.storage != "f32" else 4
    nsets = args.sets or int(min(64, max(2, -(-(1 << 30) // (set_bytes_est * main_vb // 4)) + 1)))
    runner = Runner(w, d, nsets, device, storage=args.storage, time_major=args.time_major)
    main_fmt = args.storage + (" time-major" if args.time_major else "")
    log("buffer sets: %d x %.1f MiB = %.2f GiB" % (nsets, runner.set_bytes / 2**20,
                                                    nsets * runner.set_bytes / 2**30))

    for _ in range(args.warmup):
        runner.step(names)
    torch.cuda.synchronize()

    # ---- the timed region: exactly K steps
    secs = time_region(runner, lambda: runner.step(names), args.steps)
    ms_per_step = secs / args.steps * 1e3
    value = w.E * w.T * args.steps / secs
    log("step: %.3f ms  (%.3g env-steps/s through %d estimators)" % (ms_per_step, value, len(names)))

    # ---- per-estimator back-to-back launches (same rotation), HIP events on the launch stream
    per = time_estimators(runner, names, d, w, reps)
    sweeps = {}
    nflags = int("terminated" in d) + int("truncated" in d)
    for n in names:
        mix = (PROBE_MIX[n][0], min(PROBE_MIX[n][1], nflags), PROBE_MIX[n][2])
        if mix not in sweeps:
            sweeps[mix] = None if args.no_ceiling else probe_sweep(torch, device, w.E * w.T, mix, reps)
        add_ceiling(per[n], sweeps[mix], mix)
        log_estimator(n, per[n])

    # GPU outputs for the agreement fields: (workload, host inputs, {entry: outputs}, storage format)
    checks = {main_fmt: (w, runner.host_inputs, {n: runner.outputs(n) for n in names}, args.storage)}

    # ---- the other entry points (not part of the step): the one-pass returns + TD(lambda)
    # entry and the generic episode-cut recurrence
    fused = None
    if "discounted_returns" in names and "td_lambda" in names:
        extra = ["returns_and_td_lambda", "linear_scan_segmented"]
        fused = time_estimators(runner, extra, d, w, reps)
        checks["one_pass_entries"] = (w, runner.host_inputs, {n: runner.outputs(n) for n in extra}, args.storage)
        for n in extra:
            mix = (PROBE_MIX[n][0], min(PROBE_MIX[n][1], 1 if n == "linear_scan_segmented" else nflags),
                   PROBE_MIX[n][2])
            if mix not in sweeps:
                sweeps[mix] = None if args.no_ceiling else probe_sweep(torch, device, w.E * w.T, mix, reps)
            add_ceiling(fused[n], sweeps[mix], mix)
        n = "returns_and_td_lambda"
        sep = per["discounted_returns"]["us_per_launch"] + per["td_lambda"]["us_per_launch"]
        fused[n]["separate_calls_us"] = round(sep, 3)
        fused[n]["speedup_vs_separate"] = round(sep / fused[n]["us_per_launch"], 3)
        for n in extra:
            log_estimator(n, fused[n])
        log("  (returns + td_lambda as separate calls: %.2f us)" % sep)

    # ---- vector-valued traces over [E, T, D] features (not part of the step)
    if "eligibility_traces" in names:
        vt = time_traces_vec(torch, device, reps, E=1024, T=w.T, D=64, p_term=w.p_term, p_trunc=w.p_trunc)
        fused = dict(fused or {})
        fused["eligibility_traces_vec"] = vt
        log("  %-22s %8.2f us  %7.1f GB/s  %5.1f%% of peak  (%s)" % (
            "traces, D=64", vt["us_per_launch"], vt["GBps"], 100 * vt["frac_of_peak"], vt["shape"]))

    # ---- the seven estimators with 16-bit storage and in the time-major layout
    # (not part of the step)
    variants = None
    del runner
    torch.cuda.empty_cache()
    if not args.only and not args.no_16:
        variants = {}
        for key, st, tm in (("bf16", "bf16", False), ("f16", "f16", False), ("time_major_f32", "f32", True),
                            ("time_major_bf16", "bf16", True)):
            vb = 2 if st != "f32" else 4
            nsets_v = int(min(64, max(2, -(-(1 << 30) // (set_bytes_est * vb // 4)) + 1)))
            rv = Runner(w, d, nsets_v, device, storage=st, time_major=tm)
            pv = time_estimators(rv, names, d, w, reps)
            for n in names:
                pv[n]["f32_us_per_launch"] = per[n]["us_per_launch"]
                pv[n]["speedup_vs_f32"] = round(per[n]["us_per_launch"] / pv[n]["us_per_launch"], 3)
            variants[key] = pv
            checks[key] = (w, rv.host_inputs, {n: rv.outputs(n) for n in names}, st)
            log("  %-15s " % key + "  ".join("%s %.2f us %.1f%%" % (
                n[:6], pv[n]["us_per_launch"], 100 * pv[n]["frac_of_peak"]) for n in names))
            del rv
            torch.cuda.empty_cache()

    # ---- the smaller named workloads
    configs = None
    if not args.only and not args.no_configs and w.name == "all7_16384x256":
        cfg_out = {}
        configs = run_configs(torch, device, args, reps, collect=cfg_out)
        for name, (cw, cd, outs) in cfg_out.items():
            checks["config " + name] = (cw, cd, outs, "f32")

    dom = max(per, key=lambda k: per[k]["us_per_launch"])
    traffic, traffic_src = read_traffic(dom, w.name)
    kus, kus_src = read_kernel_us(dom, w.name)
    roofline = {
        "bound": "hbm",
        "kernel": dom,
        "achieved": round(per[dom]["GBps"], 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(per[dom]["frac_of_peak"], 4),
        "traffic": traffic,
        "traffic_source": traffic_src,
        "alg_bytes_per_launch": per[dom]["alg_bytes"],
        "us_per_launch": per[dom]["us_per_launch"],
        "timing": "HIP events on the launch stream around %d back-to-back calls over rotating buffers" % reps,
        # the same kernel's average duration in the committed rocprofv3 kernel trace
        "rocprof_kernel_us": kus,
        "rocprof_frac": (round(per[dom]["alg_bytes"] / (kus * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
                         if kus else None),
        "rocprof_source": kus_src,
        # the same kernel against the fastest plain stream of its own arrays
        "ceiling": per[dom].get("ceiling"),
    }

    # ---- the oracle leg: CPU baseline and the agreement of every output above
    cpu, agreement, agree_ok = None, None, True
    if not args.no_cpu:
        log("oracle: agreement of every output ...")
        agreement = {}
        for key, (cw, cd, outs, fmt) in checks.items():
            agreement[key] = agreement_of(outs, cd, cw, fmt)
            worst = max(v["max_err"] for v in agreement[key].values())
            ok = all(v["pass"] for v in agreement[key].values())
            agree_ok = agree_ok and ok
            log("  %-28s worst %.3g  %s" % (key, worst, "ok" if ok else "FAILED"))
        checks = None
        log("cpu baseline (oracle)...")
        cpu = cpu_baseline(w, d)
        log("cpu baseline: %.3g env-steps/s on %d threads" % (cpu["value"], cpu["cores"]))

    line = {
        "metric": "env-steps/s (all seven estimators per env-step) and achieved HBM GB/s per estimator",
        "value": value,
        "unit": "env-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "storage_dtype": "%s values, u8 flags%s" % (args.storage, ", time-major" if args.time_major else ""),
        "data": "synthetic (seeded numpy draws; no dataset)",
        "config": {
            "workload": w.name, "E": w.E, "T": w.T, "estimators": names,
            "p_term": w.p_term, "p_trunc": w.p_trunc, "gamma": w.gamma, "lambda": w.lam,
            "vtrace_lambda": w.vtrace_lam, "rho_bar": w.rho_bar, "c_bar": w.c_bar,
            "buffer_sets": nsets, "gae_returns_written": False, "vtrace_pg_written": True,
            "truncation": not args.no_trunc, "calls_timed_per_estimator": reps,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": None if agreement is None else {
            "pass": agree_ok,
            "metric": "max |gpu - oracle| / max(1, |oracle|) over every element (relative where "
                      "|oracle| >= 1, absolute below); gate 1e-5, plus the storage format's unit "
                      "roundoff for 16-bit storage",
        },
        "agreement": agreement,
        "per_estimator": per,
        "one_pass_entries": fused,
        "formats_and_layouts": variants,
        "configs": configs,
        "kernel_source_sha256": kernel_source_hash(),
        "context": "rl-triton pages: 1.6-5.70x full-call speedup vs a vectorized torch.compile scan "
                   "on NVIDIA GPUs (H100 80GB HBM3, RTX 2000 Ada per the gist.science summary; the "
                   "abstract names none) - a different baseline and machine, context only",
    }
    print(json.dumps(line), flush=True)
    if not agree_ok:
        log("bench.py: GPU outputs disagree with the oracle beyond the gate")
        sys.exit(3)


if __name__ == "__main__":
    main()
