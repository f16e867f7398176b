"""GPU parity: the HIP library against the fp64 CPU oracle, element by element, on seeded inputs.

Tolerances (max-abs, after dividing by max(1, |reference|) where noted):
  * fp32 storage: 1e-5 max-abs -- the fp32 rounding of each step (~6e-8) carried through a stable
    recurrence; the kernels and the oracle see the same input bits.  The linear scan is gated on
    max-abs too (its states reach |h| ~ 10, where the relative error is printed beside it).
  * bf16 storage with fp32 arithmetic: 2e-2 is the stated bar; the inputs are the same bf16 bits on
    both sides, so the measured error is fp32-level and is also checked against 1e-4.
  * after convergence (tolerance mode) against the sequential unroll: 1e-4.
  * VJP: lambda and dL/dU relative to max(1, |ref|) <= 1e-4 (the adjoint recurrence amplifies fp32
    rounding by up to 1/(1 - max|J|)); parameter sums relative to the sum of |terms| <= 1e-5.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, dev_pre, lane_channels, max_abs, oracle_problem, sample_channels, take_channels
from nonlinear_rnn_solve_amd import api, synth

pytestmark = pytest.mark.gpu


def rel_err(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref) / np.maximum(1.0, np.abs(ref)))) if ref.size else 0.0


def announce(*a):
    print("[case]", *a, flush=True)


# ------------------------------------------------------------------------------------------------
# linear scan
# ------------------------------------------------------------------------------------------------
def stable_2x2(B, T, D, seed):
    rng = np.random.default_rng(seed)
    A = np.empty((4, B, T, D), np.float32)
    A[0] = rng.uniform(0.3, 0.9, (B, T, D))
    A[3] = rng.uniform(0.3, 0.9, (B, T, D))
    A[1] = rng.uniform(-0.1, 0.1, (B, T, D))
    A[2] = rng.uniform(-0.1, 0.1, (B, T, D))
    b = rng.standard_normal((2, B, T, D)).astype(np.float32)
    return A, b


LIN_SHAPES = [(2, 1000, 100), (1, 1, 2), (3, 257, 6), (1, 513, 130), (2, 4096, 64)]


@pytest.mark.parametrize("shape", LIN_SHAPES)
@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_linear_scan(shape, S, reverse, dtype):
    B, T, D = shape
    announce("linear_scan", shape, S, reverse, dtype)
    if S == 1:
        inp = synth.make_inputs("linear", B, T, D, dtype=dtype, seed=1100 + T)
        a, b = inp.pre
    else:
        a, b = stable_2x2(B, T, D, 1200 + T)
        if dtype == "bf16":
            a, b = synth.f32_to_bf16_bits(a), synth.f32_to_bf16_bits(b)
    s0 = synth.random_state(S, B, D, seed=7)
    odt = oracle.BF16 if dtype == "bf16" else oracle.F32
    ref = oracle.linear_scan(a, b, s0=s0, reverse=reverse, S=S, dtype=odt)
    if dtype == "bf16":
        ta = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        tb = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        ta, tb = dev(a), dev(b)
    got = api.linear_scan(ta, tb, s0=dev(s0), reverse=reverse).cpu().numpy()
    err, rel = max_abs(got, ref), rel_err(got, ref)
    print("  max abs err", err, "max rel err", rel, "max |h|", np.abs(ref).max() if ref.size else 0.0)
    assert err <= 1e-5


def test_linear_scan_in_place_and_zero_state():
    inp = synth.make_inputs("linear", 2, 3000, 64, seed=1300)
    a, b = inp.pre
    ref = oracle.linear_scan(a, b)
    ta, tb = dev(a), dev(b)
    out = api.linear_scan(ta, tb, out=tb)        # output written over b
    assert out.data_ptr() == tb.data_ptr()
    assert max_abs(out.cpu().numpy(), ref) <= 1e-5


# ------------------------------------------------------------------------------------------------
# Newton, fixed K
# ------------------------------------------------------------------------------------------------
NEWTON_CASES = [
    ("gru", "f32", (2, 1000, 200), 3),
    ("gru", "bf16", (2, 1000, 200), 3),
    ("lstm", "f32", (2, 1000, 100), 3),
    ("lstm", "bf16", (1, 777, 64), 2),
    ("linear", "f32", (2, 1000, 100), 1),
    ("linear", "bf16", (1, 300, 8), 2),
    ("gru", "f32", (1, 1, 2), 1),
    ("gru", "f32", (3, 129, 6), 5),
    ("lstm", "f32", (1, 129, 66), 4),
]


@pytest.mark.parametrize("cell,dtype,shape,K", NEWTON_CASES)
def test_newton_fixed_k(cell, dtype, shape, K):
    B, T, D = shape
    announce("newton", cell, dtype, shape, K)
    inp = synth.make_inputs(cell, B, T, D, dtype=dtype, seed=1400 + T + D)
    s0 = synth.random_state(inp.S, B, D, seed=11)
    H, res, iters, conv, rc = oracle.newton(oracle_problem(inp, s0), K)
    got, rep = api.newton_solve(cell, dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=K, s0=dev(s0))
    got = got.cpu().numpy()
    err = max_abs(got, H)
    print("  max abs err", err, "residuals gpu", rep.residuals, "oracle", list(res))
    assert rep.iters == K and not rep.converged
    assert err <= (1e-5 if dtype == "f32" else 2e-2)
    assert err <= 1e-4
    np.testing.assert_allclose(rep.residuals, res, rtol=1e-3, atol=1e-5)


def test_config0_exact_shape():
    wl = synth.WORKLOADS[0]
    announce("config0", wl.name)
    inp = synth.workload_inputs(wl)
    H, res, *_ = oracle.newton(oracle_problem(inp), wl.max_iters)
    got, rep = api.newton_solve("gru", dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=wl.max_iters)
    err = max_abs(got.cpu().numpy(), H)
    print("  max abs err", err)
    assert err <= 1e-5


# ------------------------------------------------------------------------------------------------
# Newton, warm start H^0_t = f(0, x_t)
# ------------------------------------------------------------------------------------------------
WARM_CASES = [
    ("gru", "f32", (2, 1000, 200), 1),
    ("gru", "bf16", (2, 1000, 200), 3),
    ("lstm", "f32", (2, 1000, 100), 2),
    ("lstm", "bf16", (1, 777, 64), 1),
    ("linear", "f32", (1, 300, 8), 1),
    ("gru", "f32", (1, 1, 2), 1),
    ("gru", "f32", (3, 129, 6), 2),
    ("lstm", "f32", (1, 129, 66), 3),
]


@pytest.mark.parametrize("cell,dtype,shape,K", WARM_CASES)
def test_newton_warm_start(cell, dtype, shape, K):
    B, T, D = shape
    announce("newton warm", cell, dtype, shape, K)
    inp = synth.make_inputs(cell, B, T, D, dtype=dtype, seed=1450 + T + D)
    s0 = synth.random_state(inp.S, B, D, seed=12)
    H, res, *_ = oracle.newton(oracle_problem(inp, s0), K, warm=True)
    got, rep = api.newton_solve(cell, dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=K, s0=dev(s0),
                                warm_start=True)
    err = max_abs(got.cpu().numpy(), H)
    print("  max abs err", err, "residuals gpu", rep.residuals, "oracle", list(res))
    assert err <= 1e-5 if dtype == "f32" else err <= 1e-4
    np.testing.assert_allclose(rep.residuals, res, rtol=1e-3, atol=1e-5)


def test_warm_start_is_ignored_with_an_initial_guess():
    inp = synth.make_inputs("gru", 1, 600, 16, seed=1460)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    guess, _ = api.newton_solve("gru", pre, w, b, max_iters=1)
    a, _ = api.newton_solve("gru", pre, w, b, max_iters=2, init_guess=guess.clone(), warm_start=True)
    z, _ = api.newton_solve("gru", pre, w, b, max_iters=2, init_guess=guess.clone())
    assert torch.equal(a, z)


def test_warm_start_needs_no_more_iterations():
    inp = synth.make_inputs("lstm", 2, 3000, 64, seed=1461)
    prob = oracle_problem(inp)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    _, rz = api.newton_solve("lstm", pre, w, b, max_iters=10, tol=1e-5)
    got, rw = api.newton_solve("lstm", pre, w, b, max_iters=10, tol=1e-5, warm_start=True)
    print("  zero", rz.iters, rz.residuals, "warm", rw.iters, rw.residuals)
    assert rw.converged and rw.iters <= rz.iters
    assert rw.residuals[0] < rz.residuals[0]
    assert max_abs(got.cpu().numpy(), oracle.unroll(prob)) <= 1e-4


# ------------------------------------------------------------------------------------------------
# Newton, tolerance mode
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("cell,dtype,shape", [("gru", "bf16", (1, 4096, 64)), ("gru", "f32", (2, 2000, 32)),
                                              ("lstm", "f32", (2, 2000, 32)), ("linear", "f32", (1, 5000, 16))])
def test_newton_tolerance_mode(cell, dtype, shape):
    B, T, D = shape
    announce("newton tol", cell, dtype, shape)
    inp = synth.make_inputs(cell, B, T, D, dtype=dtype, seed=1500 + T)
    prob = oracle_problem(inp)
    got, rep = api.newton_solve(cell, dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=8, tol=1e-5,
                                final_residual=True)
    got = got.cpu().numpy()
    _, ores, oit, oconv, _ = oracle.newton(prob, 8, tol=1e-5)
    print("  gpu iters", rep.iters, rep.residuals, "oracle iters", oit, list(ores))
    assert rep.converged and oconv
    assert abs(rep.iters - oit) <= 1
    H_at = oracle.newton(prob, rep.iters)[0]
    assert max_abs(got, H_at) <= 1e-4
    assert max_abs(got, oracle.unroll(prob)) <= 1e-4
    assert rep.final_residual is not None and rep.final_residual < 1e-5
    assert all(np.diff(rep.residuals[:rep.iters]) < 0)


def test_tolerance_mode_divergence_is_reported():
    inp = synth.make_inputs("gru", 1, 300, 8, seed=1600)
    inp.pre[0][0, 100, 3] = np.nan
    with pytest.raises(api.NewtonDivergenceError) as ei:
        api.newton_solve("gru", dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=6, tol=1e-5)
    assert ei.value.report.iters == 1 and np.isnan(ei.value.report.residuals[0])


def _large_weights(T, D, scale, seed):
    inp = synth.make_inputs("gru", 1, T, D, seed=seed)
    rng = np.random.default_rng(seed + 1)
    inp.w[:] = (rng.choice([-1.0, 1.0], inp.w.shape) * scale).astype(np.float32)
    return inp


@pytest.mark.parametrize("fuse", [0, 1])
def test_tolerance_mode_budget_ending_above_the_start_is_divergence(fuse):
    # recurrent weights of +-4: the first update overshoots and six iterations never bring the residual back
    # below where it started (pararnn-torch README, "Evaluation": a divergence error with the history)
    inp = _large_weights(12, 4, 4.0, 1072)
    _, ores, oit, _, orc = oracle.newton(oracle_problem(inp), 6, tol=1e-5)
    assert orc == oracle.DIVERGED and oit == 6
    with pytest.raises(api.NewtonDivergenceError) as ei:
        api.newton_solve("gru", dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=6, tol=1e-5, fuse_iters=fuse)
    rep = ei.value.report
    print("  gpu", rep.residuals, "oracle", list(ores))
    assert rep.iters == 6 and not rep.converged
    np.testing.assert_allclose(rep.residuals, ores, rtol=1e-3)
    # a fixed budget reports nothing
    _, rep0 = api.newton_solve("gru", dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=6, fuse_iters=fuse)
    assert rep0.iters == 6


def test_weights_of_fifty_diverge():
    inp = _large_weights(256, 8, 50.0, 1065)
    with pytest.raises(api.NewtonDivergenceError) as ei:
        api.newton_solve("gru", dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=6, tol=1e-5)
    rep = ei.value.report
    print("  gpu", rep.residuals)
    assert not rep.converged and not (rep.residuals[-1] <= 1e30 * rep.residuals[0])


def test_a_transient_rise_that_converges_is_not_divergence():
    inp = synth.make_inputs("lstm", 1, 1024, 8, seed=1057)
    _, ores, oit, oconv, orc = oracle.newton(oracle_problem(inp), 8, tol=1e-5)
    got, rep = api.newton_solve("lstm", dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=8, tol=1e-5)
    print("  gpu", rep.iters, rep.residuals, "oracle", oit, list(ores))
    assert orc == oracle.OK and oconv and rep.converged and rep.iters == oit
    assert rep.residuals[1] > rep.residuals[0]


def test_divergence_status_after_a_solve_without_report():
    # without a report the solve only launches; pararnn_newton_report on its workspace gives the status
    inp = _large_weights(12, 4, 4.0, 1072)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    out, r = api.newton_solve("gru", pre, w, b, max_iters=6, tol=1e-5, report=False)
    assert r is None
    lib = api.load_library()
    st = api._problem("gru", pre, w, b, None)[0]
    opts = api._Opts(6, 1e-5, None, 0, 0, 0, 0)
    nbytes = lib.pararnn_newton_workspace_bytes(ctypes.byref(st), ctypes.byref(opts))
    ws = api._workspace(nbytes, out.device, "newton")
    rep = api._Report()
    rc = lib.pararnn_newton_report(ctypes.byref(st), ctypes.byref(opts), api._ptr(out), api._ptr(ws), ws.numel(),
                                   api._stream(out.device), ctypes.byref(rep))
    assert rc == -5 and rep.iters == 6 and not rep.converged


def test_unreachable_tolerance_runs_the_budget():
    inp = synth.make_inputs("gru", 1, 500, 8, seed=1601)
    _, rep = api.newton_solve("gru", dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=3, tol=1e-30)
    assert rep.iters == 3 and not rep.converged


# ------------------------------------------------------------------------------------------------
# resume, determinism, empty problems
# ------------------------------------------------------------------------------------------------
def test_resume_equals_continuing():
    inp = synth.make_inputs("lstm", 2, 700, 34, seed=1700)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    full, _ = api.newton_solve("lstm", pre, w, b, max_iters=3)
    part, _ = api.newton_solve("lstm", pre, w, b, max_iters=2)
    api.newton_solve("lstm", pre, w, b, max_iters=1, init_guess=part, out=part)
    assert torch.equal(full, part)


def test_bitwise_determinism():
    inp = synth.make_inputs("gru", 2, 3000, 128, dtype="bf16", seed=1701, with_grad=True)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    outs = [api.newton_solve("gru", pre, w, b, max_iters=3)[0].clone() for _ in range(3)]
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    g = dev(inp.g)
    grads = [api.scan_vjp("gru", pre, outs[0], g, w, b) for _ in range(2)]
    for k in ("d_pre", "d_w", "d_bias", "d_s0"):
        assert torch.equal(grads[0][k], grads[1][k]), k
    lin = synth.make_inputs("linear", 4, 5000, 64, seed=1702)
    a, bb = dev(lin.pre[0]), dev(lin.pre[1])
    s = [api.linear_scan(a, bb).clone() for _ in range(3)]
    assert all(torch.equal(s[0], x) for x in s[1:])


def test_empty_problems_are_noops():
    z = torch.zeros(2, 0, 8, device="cuda")
    out, rep = api.newton_solve("gru", [z, z, z], torch.zeros(3, 8, device="cuda"), torch.zeros(3, 8, device="cuda"))
    assert out.shape == (1, 2, 0, 8) and rep.iters == 0
    assert api.linear_scan(z, z).shape == (2, 0, 8)


# ------------------------------------------------------------------------------------------------
# VJP
# ------------------------------------------------------------------------------------------------
VJP_CASES = [("gru", "f32", (2, 1000, 100)), ("gru", "bf16", (1, 1500, 64)), ("lstm", "f32", (2, 700, 66)),
             ("lstm", "bf16", (1, 333, 8)), ("linear", "f32", (2, 1000, 64)), ("gru", "f32", (1, 1, 2)),
             ("lstm", "f32", (1, 65, 2))]


@pytest.mark.parametrize("cell,dtype,shape", VJP_CASES)
def test_vjp(cell, dtype, shape):
    B, T, D = shape
    announce("vjp", cell, dtype, shape)
    inp = synth.make_inputs(cell, B, T, D, dtype=dtype, seed=1800 + T, with_grad=True)
    s0 = synth.random_state(inp.S, B, D, seed=13)
    prob = oracle_problem(inp, s0)
    traj = oracle.unroll(prob).astype(np.float32)           # the solved trajectory, from the oracle
    ref = oracle.vjp(prob, traj.astype(np.float64), inp.g)
    got = api.scan_vjp(cell, dev_pre(inp), dev(traj), dev(inp.g), dev(inp.w), dev(inp.bias), s0=dev(s0),
                       want_lambda=True)
    e_lam = rel_err(got["lam"].cpu().numpy(), ref["lam"])
    e_dp = rel_err(got["d_pre"].cpu().numpy(), ref["d_pre"])
    e_s0 = rel_err(got["d_s0"].cpu().numpy(), ref["d_s0"])
    print("  lambda", e_lam, "d_pre", e_dp, "d_s0", e_s0)
    assert e_lam <= 1e-4 and e_dp <= 1e-4 and e_s0 <= 1e-4
    if cell != "linear":
        # parameter sums: error relative to the sum of |terms| (|dU| times |coefficient|, summed)
        scale_b = np.abs(ref["d_pre"]).sum(axis=(1, 2)) + 1.0
        e_b = np.max(np.abs(got["d_bias"].cpu().numpy() - ref["d_bias"]) / scale_b)
        e_w = np.max(np.abs(got["d_w"].cpu().numpy() - ref["d_w"]) / (scale_b * max(1.0, np.abs(traj).max())))
        print("  d_w", e_w, "d_bias", e_b)
        assert e_w <= 1e-5 and e_b <= 1e-5


# ------------------------------------------------------------------------------------------------
# the benchmark workloads at full size: element by element where the oracle finishes in seconds
# (workloads 0-3), on sampled channels that hold every lane position of a tile for the long one (4)
# ------------------------------------------------------------------------------------------------
def test_full_config1_linear_scan():
    wl = synth.WORKLOADS[1]
    announce("full", wl.name)
    inp = synth.workload_inputs(wl)
    a, b = inp.pre
    got = api.linear_scan(dev(a), dev(b)).cpu().numpy()
    ref = oracle.linear_scan(a, b)
    err, rel = max_abs(got, ref), rel_err(got, ref)
    print("  max abs err", err, "max rel err", rel, "max |h|", np.abs(ref).max())
    assert err <= 1e-5


@pytest.mark.parametrize("idx", [2, 3])
def test_full_config_newton(idx):
    wl = synth.WORKLOADS[idx]
    announce("full", wl.name)
    inp = synth.workload_inputs(wl)
    got, rep = api.newton_solve(wl.cell, dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=wl.max_iters)
    got = got.cpu().numpy()
    H, res, *_ = oracle.newton(oracle_problem(inp), wl.max_iters)
    err = max_abs(got, H)
    print("  max abs err (every element)", err, "gpu residuals", rep.residuals, "oracle", list(res))
    assert err <= (1e-5 if wl.dtype == "f32" else 2e-2)
    assert err <= 1e-4
    np.testing.assert_allclose(rep.residuals, res, rtol=1e-3, atol=1e-5)


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_full_size_vjp_at_the_fixed_budget_workloads(idx):
    # these workloads time no VJP; here the VJP kernels run at their full shapes (the linear scan's, the GRU's
    # with bf16 gate inputs, the LSTM's): at the GPU's converged trajectory against the oracle's adjoint at that same trajectory, on sampled
    # channels that hold every lane position of a tile (the gradient drawn after the workload's other inputs)
    wl = synth.WORKLOADS[idx]
    announce("full vjp", wl.name)
    inp = synth.make_inputs(wl.cell, wl.B, wl.T, wl.D, dtype=wl.dtype, seed=wl.index, with_grad=True)
    pre = dev_pre(inp)
    w, b = (None, None) if inp.w is None else (dev(inp.w), dev(inp.bias))
    got, rep = api.newton_solve(wl.cell, pre, w, b, max_iters=8, tol=1e-5)
    assert rep.converged
    gr = api.scan_vjp(wl.cell, pre, got, dev(inp.g), w, b, want_lambda=True)
    ch = lane_channels(wl.B, wl.D, 8, seed=7)
    prob = oracle_problem(inp, channels=ch)
    g_s = take_channels(got.cpu().numpy(), ch)
    ref = oracle.vjp(prob, g_s.astype(np.float64), take_channels(inp.g, ch))
    e_lam = rel_err(take_channels(gr["lam"].cpu().numpy(), ch), ref["lam"])
    e_dp = rel_err(take_channels(gr["d_pre"].cpu().numpy(), ch), ref["d_pre"])
    print("  iters", rep.iters, "vjp lambda", e_lam, "d_pre", e_dp)
    assert e_lam <= 1e-4 and e_dp <= 1e-4


@pytest.mark.parametrize("idx", [0, 2, 3])
def test_full_config_after_convergence(idx):
    # the tolerance-mode run of each fixed-budget workload (tol 1e-5, at most 8 iterations): every element
    # within 1e-4 of the sequential unroll, the oracle's iterate at the GPU's count, the oracle's own count
    # within one of the GPU's
    wl = synth.WORKLOADS[idx]
    announce("full after convergence", wl.name)
    inp = synth.workload_inputs(wl)
    prob = oracle_problem(inp)
    got, rep = api.newton_solve(wl.cell, dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=8, tol=1e-5,
                                final_residual=True)
    got = got.cpu().numpy()
    H, ores, oit, oconv, orc = oracle.newton(prob, 8, tol=1e-5)
    print("  gpu iters", rep.iters, rep.residuals, "final", rep.final_residual, "oracle iters", oit, list(ores))
    assert rep.converged and oconv and orc == oracle.OK
    assert abs(rep.iters - oit) <= 1
    if rep.iters != oit:
        H = oracle.newton(prob, rep.iters)[0]
    e_it = max_abs(got, H)
    del H
    e_un = max_abs(got, oracle.unroll(prob))
    print("  vs oracle iterate", e_it, "vs unroll", e_un)
    assert e_it <= (1e-5 if wl.dtype == "f32" else 1e-4)
    assert e_un <= 1e-4
    assert rep.final_residual < 1e-5


def test_full_config4_newton_tol_and_vjp():
    wl = synth.WORKLOADS[4]
    announce("full", wl.name)
    inp = synth.workload_inputs(wl)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    got, rep = api.newton_solve("gru", pre, w, b, max_iters=wl.max_iters, tol=wl.tol, final_residual=True)
    print("  iters", rep.iters, rep.residuals)
    assert rep.converged and rep.final_residual < wl.tol
    # the launch configuration the benchmark times (the solve's iteration count in one fused launch): the
    # same bits and the same report as the library's default launch length checked below
    got_b, rep_b = api.newton_solve("gru", pre, w, b, max_iters=wl.max_iters, tol=wl.tol, final_residual=True,
                                    fuse_iters=rep.iters)
    assert torch.equal(got_b, got) and rep_b.iters == rep.iters and rep_b.residuals == rep.residuals
    del got_b
    ch = lane_channels(wl.B, wl.D, 16, seed=3)
    prob = oracle_problem(inp, channels=ch)
    H, ores, oit, oconv, _ = oracle.newton(prob, wl.max_iters, tol=wl.tol)
    print("  oracle on the sample: iters", oit, list(ores))
    # the sample's max residual is at most the whole problem's, so its count can only be lower
    assert oconv and rep.iters - 1 <= oit <= rep.iters
    if oit != rep.iters:
        H = oracle.newton(prob, rep.iters)[0]
    unroll = oracle.unroll(prob)
    g_s = take_channels(got.cpu().numpy(), ch)
    print("  vs oracle iterate", max_abs(g_s, H), "vs unroll", max_abs(g_s, unroll))
    assert max_abs(g_s, H) <= 1e-4 and max_abs(g_s, unroll) <= 1e-4
    # VJP at the GPU's converged trajectory vs the oracle's adjoint at the exact (unrolled) solution
    gt = dev(inp.g)
    gr = api.scan_vjp("gru", pre, got, gt, w, b, want_lambda=True)
    ref = oracle.vjp(prob, unroll, take_channels(inp.g, ch))
    e_lam = rel_err(take_channels(gr["lam"].cpu().numpy(), ch), ref["lam"])
    e_dp = rel_err(take_channels(gr["d_pre"].cpu().numpy(), ch), ref["d_pre"])
    ds = np.array([c[1] for c in ch])
    e_dw = np.max(np.abs(gr["d_w"].cpu().numpy()[:, ds] - ref["d_w"]) / (1 + np.abs(ref["d_w"])))
    print("  vjp lambda", e_lam, "d_pre", e_dp, "d_w", e_dw)
    assert e_lam <= 2e-2 and e_dp <= 2e-2 and e_dw <= 2e-2
    # and the VJP at the GPU's own trajectory against the oracle's adjoint at that same trajectory
    ref_g = oracle.vjp(prob, g_s.astype(np.float64), take_channels(inp.g, ch))
    e_lam = rel_err(take_channels(gr["lam"].cpu().numpy(), ch), ref_g["lam"])
    e_dp = rel_err(take_channels(gr["d_pre"].cpu().numpy(), ch), ref_g["d_pre"])
    print("  vjp at the same trajectory: lambda", e_lam, "d_pre", e_dp)
    assert e_lam <= 1e-4 and e_dp <= 1e-4


# ------------------------------------------------------------------------------------------------
# automatic budget K*(T) (max_iters = 0): the measured table against the sequential unroll
# ------------------------------------------------------------------------------------------------
def _kstar_gold():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "kstar.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("cell,T,warm", [("gru", 16384, False), ("gru", 16384, True), ("lstm", 4096, False),
                                         ("lstm", 16384, True), ("gru", 131072, False), ("lstm", 131072, True)])
def test_automatic_budget_meets_the_agreement_tolerance(cell, T, warm):
    gold = _kstar_gold()
    e = [x for x in gold["entries"] if x["cell"] == cell and x["T"] == T and x["init"] == ("warm" if warm else "zero")][0]
    announce("auto budget", cell, T, "warm" if warm else "zero", "K*", e["kstar"])
    inp = synth.make_inputs(cell, gold["B"], T, gold["D"], dtype=e["dtype"], seed=e["seed"])
    got, rep = api.newton_solve(cell, dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=None, warm_start=warm)
    assert rep.iters == e["kstar"] == api.newton_budget(cell, T, warm)
    # the full trajectory up to 16384 steps, sampled channels beyond
    ch = None if T <= 16384 else sample_channels(gold["B"], gold["D"], 24, seed=5)
    prob = oracle_problem(inp, channels=ch)
    g = got.cpu().numpy() if ch is None else take_channels(got.cpu().numpy(), ch)
    err_unroll = max_abs(g, oracle.unroll(prob))
    err_iter = max_abs(g, oracle.newton(prob, e["kstar"], warm=warm)[0])
    print("  vs unroll", err_unroll, "vs oracle iterate", err_iter)
    assert err_iter <= 1e-5
    assert err_unroll <= gold["tau"] + 1e-5
