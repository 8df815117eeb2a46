"""GPU invariants that hold at any size (bitwise where the arithmetic allows).

* run-to-run determinism (bitwise);
* permuting env rows permutes outputs (bitwise);
* episode isolation: changing the inputs of one episode leaves every output of
  the other episodes bit-identical (a cut enters the scan as an exact zero);
* chaining two windows of a forward estimator through `init` equals one call;
* the generic recurrence: reverse scan == forward scan of flipped arrays, and
  parity with the oracle;
* calls on a side stream and inside a captured HIP graph (replayed several
  times) match eager calls.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from linear_recurrence_scan_reverse_amd import synth
from tests.estimators import NAMES, TOL, parity_err, run_gpu, to_dev

pytestmark = pytest.mark.gpu


def _np(out):
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("T", [64, 256, 1000])
def test_bitwise_determinism(T):
    d = synth.draw(300, T, seed=21, p_term=0.01, p_trunc=0.01)
    dd = to_dev(d)
    for name in NAMES:
        a = _np(run_gpu(name, dd))
        b = _np(run_gpu(name, dd))
        for k in a:
            assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), (name, k)


@pytest.mark.parametrize("T", [64, 128, 256, 777])
def test_row_permutation_equivariance(T):
    E = 97
    d = synth.draw(E, T, seed=22, p_term=0.02, p_trunc=0.02)
    perm = np.random.default_rng(5).permutation(E)
    dp = {k: np.ascontiguousarray(v[perm]) for k, v in d.items()}
    base = {n: _np(run_gpu(n, to_dev(d))) for n in NAMES}
    moved = {n: _np(run_gpu(n, to_dev(dp))) for n in NAMES}
    for n in NAMES:
        for k in base[n]:
            assert np.array_equal(base[n][k][perm].view(np.uint32), moved[n][k].view(np.uint32)), (n, k)


@pytest.mark.parametrize("T,j", [(256, 100), (256, 3), (1024, 700), (64, 40)])
def test_episode_isolation_bitwise(T, j):
    """Row 5 terminates at step j: later inputs never reach earlier outputs and vice versa."""
    E, e = 16, 5
    d = synth.draw(E, T, seed=23, p_term=0.0, p_trunc=0.0)
    d["terminated"][e, j] = 1
    base = {n: _np(run_gpu(n, to_dev(d))) for n in NAMES}

    later = {k: v.copy() for k, v in d.items()}
    for k in ("r", "v", "log_rhos", "q", "exp_q", "trunc_bootstrap"):
        later[k][e, j + 1:] += 3.5
    later["pi"][e, j + 1:] *= 0.5
    # (bootstrap_value is left alone: the forward estimators take it as init, which
    # belongs to the earlier episode)
    after = {n: _np(run_gpu(n, to_dev(later))) for n in NAMES}
    for n in NAMES:
        for k in base[n]:
            assert np.array_equal(base[n][k][e, :j + 1].view(np.uint32),
                                  after[n][k][e, :j + 1].view(np.uint32)), ("later->earlier", n, k)
            other = np.arange(E) != e
            assert np.array_equal(base[n][k][other].view(np.uint32), after[n][k][other].view(np.uint32))

    earlier = {k: v.copy() for k, v in d.items()}
    for k in ("r", "v", "log_rhos", "q", "exp_q", "trunc_bootstrap"):
        earlier[k][e, :j + 1] -= 1.25
    earlier["mu"][e, :j + 1] *= 0.5
    after = {n: _np(run_gpu(n, to_dev(earlier))) for n in NAMES}
    for n in NAMES:
        for k in base[n]:
            assert np.array_equal(base[n][k][e, j + 1:].view(np.uint32),
                                  after[n][k][e, j + 1:].view(np.uint32)), ("earlier->later", n, k)


def test_forward_windows_chain_through_init():
    """Two windows chained with init = last output (zeroed after a done) == one call."""
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    rng = np.random.default_rng(24)
    E, T, T1 = 40, 600, 257
    x = rng.integers(-20, 21, size=(E, T)).astype(np.float32)
    term = (rng.random((E, T)) < 0.01).astype(np.uint8)
    xd, td = torch.from_numpy(x).cuda(), torch.from_numpy(term).cuda()
    full = rl.episodic_prefix_sum(xd, td)
    first = rl.episodic_prefix_sum(xd[:, :T1].contiguous(), td[:, :T1].contiguous())
    init = torch.where(td[:, T1 - 1] != 0, torch.zeros_like(first[:, -1]), first[:, -1]).contiguous()
    second = rl.episodic_prefix_sum(xd[:, T1:].contiguous(), td[:, T1:].contiguous(), init=init)
    assert torch.equal(torch.cat([first, second], 1), full)
    tr_full = rl.eligibility_traces(xd, td, gamma=0.9, lam=0.8)
    tr1 = rl.eligibility_traces(xd[:, :T1].contiguous(), td[:, :T1].contiguous(), gamma=0.9, lam=0.8)
    init = torch.where(td[:, T1 - 1] != 0, torch.zeros_like(tr1[:, -1]), tr1[:, -1]).contiguous()
    tr2 = rl.eligibility_traces(xd[:, T1:].contiguous(), td[:, T1:].contiguous(), init=init, gamma=0.9, lam=0.8)
    # the chained result rounds the carry to fp32 once at the window edge
    assert parity_err(torch.cat([tr1, tr2], 1).cpu().numpy(), tr_full.cpu().numpy()) <= TOL


@pytest.mark.parametrize("T", [1, 5, 64, 65, 256, 999, 4100])
def test_generic_scan_parity_and_mirror(T):
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    rng = np.random.default_rng(25 + T)
    E = 21
    a = rng.uniform(-1.0, 1.0, size=(E, T)).astype(np.float32)
    b = rng.standard_normal((E, T)).astype(np.float32)
    c = rng.standard_normal(E).astype(np.float32)
    ad, bd, cd = (torch.from_numpy(v).cuda() for v in (a, b, c))
    for rev in (True, False):
        got = rl.linear_scan(ad, bd, cd, reverse=rev).cpu().numpy()
        assert parity_err(got, oracle.linear_scan(a, b, c, reverse=rev)) <= TOL
    rev = rl.linear_scan(ad, bd, cd, reverse=True)
    fwd_flipped = rl.linear_scan(ad.flip(1).contiguous(), bd.flip(1).contiguous(), cd, reverse=False)
    assert parity_err(fwd_flipped.flip(1).cpu().numpy(), rev.cpu().numpy()) <= TOL


def test_generic_scan_special_cases():
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    rng = np.random.default_rng(26)
    E, T = 7, 300
    b = torch.from_numpy(rng.standard_normal((E, T)).astype(np.float32)).cuda()
    c = torch.from_numpy(rng.standard_normal(E).astype(np.float32)).cuda()
    zeros, ones = torch.zeros_like(b), torch.ones_like(b)
    for rev in (True, False):
        assert torch.equal(rl.linear_scan(zeros, b, c, reverse=rev), b)
        assert torch.equal(rl.linear_scan(ones, zeros, c, reverse=rev), c[:, None].expand(E, T))


def test_side_stream_and_graph_capture():
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    d = synth.draw(512, 256, seed=27, p_term=0.01, p_trunc=0.01)
    dd = to_dev(d)
    eager = _np(run_gpu("gae", dd))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        side = _np(run_gpu("gae", dd))
    torch.cuda.current_stream().wait_stream(s)
    for k in eager:
        assert np.array_equal(eager[k], side[k])

    adv = torch.empty_like(dd["r"])
    ret = torch.empty_like(dd["r"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rl.gae(dd["r"], dd["v"], dd["terminated"], dd["truncated"], dd["bootstrap_value"],
               dd["trunc_bootstrap"], advantages=adv, returns=ret)
    for rep in range(4):
        adv.fill_(float("nan"))
        ret.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(adv.cpu().numpy(), eager["out"]), rep
        assert np.array_equal(ret.cpu().numpy(), eager["out1"]), rep


@pytest.mark.parametrize("T", [1, 5, 64, 65, 256, 257, 1000, 4100])
@pytest.mark.parametrize("p_cut", [0.0, 0.05, 0.5])
def test_segmented_generic_scan_parity(T, p_cut):
    """The episode-cut generic recurrence against the oracle, both directions,
    with and without a carry, and equal to the plain recurrence when nothing is cut."""
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    rng = np.random.default_rng(60 + T)
    E = 21
    a = rng.uniform(-1.0, 1.0, size=(E, T)).astype(np.float32)
    b = rng.standard_normal((E, T)).astype(np.float32)
    c = rng.standard_normal(E).astype(np.float32)
    done = (rng.random((E, T)) < p_cut).astype(np.uint8)
    ad, bd, cd, dd = (torch.from_numpy(v).cuda() for v in (a, b, c, done))
    for rev in (True, False):
        for carry, cdev in ((None, None), (c, cd)):
            got = rl.linear_scan_segmented(ad, bd, dd, cdev, reverse=rev).cpu().numpy()
            assert parity_err(got, oracle.linear_scan_segmented(a, b, done, carry, reverse=rev)) <= TOL
        plain = rl.linear_scan(ad, bd, cd, reverse=rev)
        uncut = rl.linear_scan_segmented(ad, bd, None, cd, reverse=rev)
        assert torch.equal(plain, uncut)


def test_segmented_generic_scan_long_rows_and_exact_sums():
    """Long rows (the segmented three-pass path) and exact integer episode sums."""
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    rng = np.random.default_rng(61)
    E, T = 3, 50000
    a = rng.uniform(-1.0, 1.0, size=(E, T)).astype(np.float32)
    b = rng.standard_normal((E, T)).astype(np.float32)
    done = (rng.random((E, T)) < 0.001).astype(np.uint8)
    ad, bd, dd = (torch.from_numpy(v).cuda() for v in (a, b, done))
    for rev in (True, False):
        got = rl.linear_scan_segmented(ad, bd, dd, None, reverse=rev).cpu().numpy()
        assert parity_err(got, oracle.linear_scan_segmented(a, b, done, None, reverse=rev)) <= TOL
    ones = np.ones((E, T), dtype=np.float32)
    bi = rng.integers(-5, 6, size=(E, T)).astype(np.float32)
    for rev in (True, False):
        got = rl.linear_scan_segmented(torch.from_numpy(ones).cuda(), torch.from_numpy(bi).cuda(), dd, None,
                                       reverse=rev).cpu().numpy()
        assert np.array_equal(got.astype(np.float64),
                              oracle.linear_scan_segmented(ones, bi, done, None, reverse=rev))


def test_graph_capture_of_formats_layouts_and_long_rows():
    # a captured HIP graph holding a time-major bfloat16 call, a row-major
    # float16 call, a segmented long-row call and a time-major float32 call in
    # the item form (six kernels), replayed several times with the program's
    # own work between replays: every replay matches the eager result bit for
    # bit
    import torch
    import linear_recurrence_scan_reverse_amd as rl
    from tests.estimators import storage_inputs
    d1 = synth.draw(300, 200, seed=28, p_term=0.01, p_trunc=0.01)
    _, tm = storage_inputs(d1, "bfloat16", time_major=True)
    _, hf = storage_inputs(d1, "float16")
    d2 = synth.draw(2, 40000, seed=29, p_term=0.001, p_trunc=0.001)
    lr = to_dev(d2)
    d3 = synth.draw(256, 320, seed=30, p_term=0.01, p_trunc=0.01)
    _, ti = storage_inputs(d3, "float32", time_major=True)

    def calls(outs):
        rl.gae(tm["r"], tm["v"], tm["terminated"], tm["truncated"], tm["bootstrap_value"], tm["trunc_bootstrap"],
               time_major=True, advantages=outs[0], returns=outs[1])
        rl.retrace(hf["r"], hf["q"], hf["exp_q"], hf["pi"], hf["mu"], hf["terminated"], hf["truncated"],
                   hf["bootstrap_value"], hf["trunc_bootstrap"], out=outs[2])
        rl.discounted_returns(lr["r"], lr["terminated"], lr["truncated"], lr["bootstrap_value"],
                              lr["trunc_bootstrap"], out=outs[3])
        rl.vtrace(ti["r"], ti["v"], ti["log_rhos"], ti["terminated"], ti["truncated"], ti["bootstrap_value"],
                  ti["trunc_bootstrap"], time_major=True, vs=outs[4], pg_advantages=outs[5])

    def fresh():
        return [torch.empty_like(tm["r"]), torch.empty_like(tm["r"]), torch.empty_like(hf["r"]),
                torch.empty_like(lr["r"]), torch.empty_like(ti["r"]), torch.empty_like(ti["r"])]

    eager = fresh()
    calls(eager)
    torch.cuda.synchronize()
    eager = [x.cpu() for x in eager]
    outs = fresh()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(outs)
    for rep in range(3):
        for x in outs:
            x.fill_(float("nan"))
        calls(fresh())  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a.cpu().view(torch.int16) if a.element_size() == 2 else a.cpu(),
                               b.view(torch.int16) if b.element_size() == 2 else b), rep


def test_concurrent_host_threads():
    # the library keeps no state between calls (a per-device compute-unit count
    # aside): four host threads, each on its own stream, calling different
    # estimators and formats at once give the single-threaded results bit for bit
    import threading

    import torch
    from tests.estimators import storage_inputs
    d = synth.draw(704, 256, seed=31, p_term=0.01, p_trunc=0.01)
    jobs = [("gae", "float32", False), ("retrace", "float32", False), ("vtrace", "bfloat16", False),
            ("td_lambda", "float16", True)]  # the last in the time-major item form (704 = 22 x 32)
    inputs = [storage_inputs(d, fmt, time_major=tm)[1] for _, fmt, tm in jobs]

    def raw(outs):
        return {k: v.cpu().view(torch.int16 if v.element_size() == 2 else torch.int32) for k, v in outs.items()}

    ref = [raw(run_gpu(name, dev, time_major=tm)) for (name, _, tm), dev in zip(jobs, inputs)]
    torch.cuda.synchronize()
    results = [None] * len(jobs)
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = None
                for _ in range(20):
                    outs = run_gpu(jobs[i][0], inputs[i], time_major=jobs[i][2])
                s.synchronize()
                results[i] = raw(outs)
        except Exception as ex:  # reported below
            errors.append(repr(ex))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i, (r, g) in enumerate(zip(ref, results)):
        for k in r:
            assert torch.equal(r[k], g[k]), (jobs[i], k)


@pytest.mark.parametrize("T", [128, 256, 512, 1024])
def test_zero_flag_arrays_match_absent_flags(T):
    """All-zero flag arrays and absent (NULL) flags describe the same episodes, but
    a call with flag arrays runs other template instances than one without
    (they read and decode the flag bytes, and the backward estimators gather
    truncation bootstraps).  Each pair must agree to fp32 rounding of the same
    fp64 result; no oracle is involved."""
    E = 2048
    d = synth.draw(E, T, seed=500 + T, p_term=0.0, p_trunc=0.0)
    assert not d["terminated"].any() and not d["truncated"].any()
    dd = to_dev(d)
    for name in NAMES:
        with_flags = _np(run_gpu(name, dd))
        without = _np(run_gpu(name, dd, term=False, trunc=False))
        for k in with_flags:
            err = parity_err(with_flags[k], without[k])
            assert err <= 1e-6, "%s %s T=%d: zero flags vs no flags differ by %.3g" % (name, k, T, err)
