"""GPU parity for the diagonal sLSTM (state c, n, m, h; gates z, i, f, o) and for Picard sweeps:
the HIP library against the fp64 oracle on the same seeded inputs.

Tolerances: the cell's exponential gates make fp32 rounding grow through the Newton iterates, so
iterates are compared relative to max(1, |ref|) at 1e-4 (fp32 storage) and 2e-3 (bf16 storage of
the gate inputs, same bits on both sides); converged results against the fp64 unroll at 1e-4; the
VJP at 1e-4 relative, parameter sums at 1e-5 of the sum of |terms| (as for the other cells).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, dev_pre, lane_channels, max_abs, oracle_problem, sample_channels, take_channels
from nonlinear_rnn_solve_amd import api, synth

pytestmark = pytest.mark.gpu


def announce(*a):
    print("[case]", *a, flush=True)


def rel_err(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref) / np.maximum(1.0, np.abs(ref)))) if ref.size else 0.0


def positive_state(S, B, D, seed):
    s0 = synth.random_state(S, B, D, seed=seed)
    s0[1] = np.abs(s0[1]) + 0.5     # the normaliser n is positive
    return s0


CASES = [("f32", (2, 1000, 64), 8, 12, False), ("bf16", (1, 3000, 32), 8, 14, False),
         ("f32", (3, 129, 6), 2, 6, True), ("f32", (1, 1, 2), 0, 1, False), ("f32", (2, 500, 18), 5, 5, False)]


@pytest.mark.parametrize("dtype,shape,P,K,warm", CASES)
def test_slstm_newton_with_picard(dtype, shape, P, K, warm):
    B, T, D = shape
    announce("slstm newton", dtype, shape, "picard", P, "K", K, "warm" if warm else "zero")
    inp = synth.make_inputs("slstm", B, T, D, dtype=dtype, seed=2800 + T + D)
    s0 = positive_state(4, B, D, seed=50)
    prob = oracle_problem(inp, s0)
    H, res, *_ = oracle.newton(prob, K, picard=P, warm=warm)
    got, rep = api.newton_solve("slstm", dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=K, s0=dev(s0),
                                picard_iters=P, warm_start=warm)
    err = rel_err(got.cpu().numpy(), H)
    print("  rel err", err, "residuals gpu", rep.residuals, "oracle", list(res))
    assert err <= (1e-4 if dtype == "f32" else 2e-3)
    np.testing.assert_allclose(rep.residuals, res, rtol=1e-3, atol=1e-5)


def test_slstm_tolerance_mode_reaches_the_unroll():
    inp = synth.make_inputs("slstm", 2, 4000, 32, seed=2810)
    prob = oracle_problem(inp)
    got, rep = api.newton_solve("slstm", dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=24, tol=1e-5,
                                picard_iters=8, final_residual=True)
    print("  iters", rep.iters, rep.residuals, "final", rep.final_residual)
    assert rep.converged and rep.final_residual < 1e-4
    assert max_abs(got.cpu().numpy(), oracle.unroll(prob)) <= 1e-4


@pytest.mark.parametrize("T", [1024, 4096])
def test_slstm_tolerance_count_equals_the_oracle_on_the_whole_problem(T):
    # the README's sLSTM benchmark shape (B = 8, D = 256) at T = 1024 and 4096 (the inputs the sLSTM benchmark
    # times): 8 Picard sweeps, then Newton to 1e-5.  The count is set by the slowest of the 2048 channels, so
    # it is compared with the fp64 oracle on every channel (a sample of channels converges sooner), and so is
    # the iterate.  At T = 4096 both need 21 updates: Newton's transient after the sweeps, not fp32 rounding
    # near tol, sets the count (the fp64 history ends 1e-3, 5e-8)
    announce("slstm tolerance count", "f32", (8, T, 256))
    inp = synth.make_inputs("slstm", 8, T, 256, seed=4000 + T // 1024)
    prob = oracle_problem(inp)
    H, ores, oit, oconv, _ = oracle.newton(prob, 40, tol=1e-5, picard=8)
    got, rep = api.newton_solve("slstm", dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=40, tol=1e-5,
                                picard_iters=8)
    print("  gpu iters", rep.iters, rep.residuals[8:], "oracle iters", oit, list(ores[8:]))
    assert rep.converged and oconv and rep.iters == oit
    assert rel_err(got.cpu().numpy(), H) <= 1e-4


def test_slstm_full_size_tolerance_solve_and_vjp():
    # the largest shape the sLSTM benchmark times (B = 8, T = 65536, D = 256), in its launch configuration: the
    # tolerance-mode solve against the fp64 unroll, and the VJP at the GPU's trajectory against the oracle's
    # adjoint at that same trajectory, on sampled channels that hold every lane position of a tile
    B, T, D = 8, 65536, 256
    announce("slstm full size", (B, T, D))
    inp = synth.make_inputs("slstm", B, T, D, seed=4000 + T // 1024, with_grad=True)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    got, rep = api.newton_solve("slstm", pre, w, b, max_iters=40, tol=1e-5, picard_iters=8, final_residual=True)
    print("  iters", rep.iters, "final residual", rep.final_residual)
    assert rep.converged and rep.final_residual < 1e-4
    gr = api.scan_vjp("slstm", pre, got, dev(inp.g), w, b, want_lambda=True)
    ch = lane_channels(B, D, 8, seed=6)
    prob = oracle_problem(inp, channels=ch)
    g_s = take_channels(got.cpu().numpy(), ch)
    e_un = max_abs(g_s, oracle.unroll(prob))
    ref = oracle.vjp(prob, g_s.astype(np.float64), take_channels(inp.g, ch))
    e_lam = rel_err(take_channels(gr["lam"].cpu().numpy(), ch), ref["lam"])
    e_dp = rel_err(take_channels(gr["d_pre"].cpu().numpy(), ch), ref["d_pre"])
    print("  vs unroll", e_un, "vjp lambda", e_lam, "d_pre", e_dp)
    assert e_un <= 1e-4 and e_lam <= 1e-4 and e_dp <= 1e-4


def test_slstm_tolerance_launches_on_a_resident_grid_give_the_same_bits():
    # in tolerance mode the late Newton iterations of a cell without a fused pass run on a grid of what is
    # resident, each workgroup taking several tiles (here 1024 tiles); the trajectory must equal that of the
    # same number of iterations at a fixed budget (one workgroup per tile) bit for bit.  This input takes 21
    # updates, so its last one runs on the resident grid while it still works, and the 19 after it find the
    # solve stopped
    announce("slstm resident-grid launches", "f32", (8, 4096, 256))
    inp = synth.make_inputs("slstm", 8, 4096, 256, seed=4004)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    got, rep = api.newton_solve("slstm", pre, w, b, max_iters=40, tol=1e-5, picard_iters=8)
    assert rep.converged and rep.iters > 20
    fixed, rep_f = api.newton_solve("slstm", pre, w, b, max_iters=rep.iters, picard_iters=8)
    assert torch.equal(got, fixed)
    np.testing.assert_array_equal(rep.residuals, rep_f.residuals[:rep.iters])


@pytest.mark.parametrize("dtype,shape", [("f32", (2, 700, 40)), ("bf16", (1, 1200, 16)), ("f32", (1, 65, 2)),
                                         ("f32", (3, 1, 6)), ("f32", (1, 97, 34)), ("f32", (2, 193, 64))])
def test_slstm_vjp(dtype, shape):
    B, T, D = shape
    announce("slstm vjp", dtype, shape)
    inp = synth.make_inputs("slstm", B, T, D, dtype=dtype, seed=2820 + T, with_grad=True)
    s0 = positive_state(4, B, D, seed=51)
    prob = oracle_problem(inp, s0)
    traj = oracle.unroll(prob).astype(np.float32)
    ref = oracle.vjp(prob, traj.astype(np.float64), inp.g)
    got = api.scan_vjp("slstm", dev_pre(inp), dev(traj), dev(inp.g), dev(inp.w), dev(inp.bias), s0=dev(s0),
                       want_lambda=True)
    e_lam = rel_err(got["lam"].cpu().numpy(), ref["lam"])
    e_dp = rel_err(got["d_pre"].cpu().numpy(), ref["d_pre"])
    e_s0 = rel_err(got["d_s0"].cpu().numpy(), ref["d_s0"])
    scale_b = np.abs(ref["d_pre"]).sum(axis=(1, 2)) + 1.0
    e_b = np.max(np.abs(got["d_bias"].cpu().numpy() - ref["d_bias"]) / scale_b)
    e_w = np.max(np.abs(got["d_w"].cpu().numpy() - ref["d_w"]) / (scale_b * max(1.0, np.abs(traj[3]).max())))
    print("  lambda", e_lam, "d_pre", e_dp, "d_s0", e_s0, "d_w", e_w, "d_bias", e_b)
    assert e_lam <= 1e-4 and e_dp <= 1e-4 and e_s0 <= 1e-4
    assert e_w <= 1e-5 and e_b <= 1e-5


def test_slstm_packed_sequences():
    inp = synth.make_inputs("slstm", 2, 900, 16, seed=2830, with_grad=True)
    cu = synth.packed_offsets(900, 2831, 150, forced=(1, 64, 65, 128, 899))
    tcu = torch.from_numpy(cu).cuda()
    prob = oracle_problem(inp, cu_seqlens=cu)
    H, res, *_ = oracle.newton(prob, 10, picard=6)
    got, rep = api.newton_solve("slstm", dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=10, picard_iters=6,
                                cu_seqlens=tcu)
    err = rel_err(got.cpu().numpy(), H)
    print("  n_seqs", len(cu) - 1, "rel err", err)
    assert err <= 1e-4
    traj = oracle.unroll(prob).astype(np.float32)
    ref = oracle.vjp(prob, traj.astype(np.float64), inp.g)
    gr = api.scan_vjp("slstm", dev_pre(inp), dev(traj), dev(inp.g), dev(inp.w), dev(inp.bias), want_lambda=True,
                      cu_seqlens=tcu)
    assert rel_err(gr["lam"].cpu().numpy(), ref["lam"]) <= 1e-4
    assert rel_err(gr["d_pre"].cpu().numpy(), ref["d_pre"]) <= 1e-4


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_picard_sweeps_on_the_other_cells(cell):
    inp = synth.make_inputs(cell, 2, 800, 34, seed=2840)
    s0 = synth.random_state(inp.S, 2, 34, seed=52)
    prob = oracle_problem(inp, s0)
    for P, K in ((3, 3), (2, 5)):
        H, res, *_ = oracle.newton(prob, K, picard=P)
        got, rep = api.newton_solve(cell, dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=K, s0=dev(s0),
                                    picard_iters=P)
        err = max_abs(got.cpu().numpy(), H)
        print("  P", P, "K", K, "max abs err", err)
        assert err <= 1e-5
        np.testing.assert_allclose(rep.residuals, res, rtol=1e-3, atol=1e-5)
